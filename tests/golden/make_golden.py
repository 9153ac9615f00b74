"""Write tests/golden/oracle_tiny.json: the fp64 oracle's output on one tiny seeded case.

Regression fixture for the oracle (and a fixed target for the HIP path). It is written
by this script from the oracle alone; rerun it only when the oracle's arithmetic changes
for a reason that cites the pages.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from decode_attention_gather_amd import inputs  # noqa: E402

CASE = dict(kv_lens=[5, 40, 67], num_heads=2, q_len=2, seed=31337, output_scale=1.25)


def make_case():
    kw = dict(CASE)
    lens = kw.pop("kv_lens")
    return inputs.make_case(lens, **kw)


def compute():
    case = make_case()
    o, lse = oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens,
                               q_len=case.q_len, num_heads=case.num_heads,
                               softmax_scale=float(np.float32(case.softmax_scale)),
                               output_scale=case.output_scale)
    return case, o, lse


if __name__ == "__main__":
    case, o, lse = compute()
    out = {
        "what": "fp64 oracle output on a seeded tiny case (see make_golden.py)",
        "case": CASE,
        "softmax_scale_f32": float(np.float32(case.softmax_scale)),
        "lse": [float(x) for x in lse],
        "o_first16": [[float(x) for x in row[:16]] for row in o],
        "o_sum": [float(x) for x in o.sum(axis=1)],
    }
    with open(os.path.join(HERE, "oracle_tiny.json"), "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", os.path.join(HERE, "oracle_tiny.json"))
