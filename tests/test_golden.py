"""The oracle still reproduces its stored output on the tiny seeded case."""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_matches_golden():
    gold = json.load(open(os.path.join(HERE, "golden", "oracle_tiny.json")))
    _, o, lse = make_golden.compute()
    np.testing.assert_allclose(lse, gold["lse"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o[:, :16], np.array(gold["o_first16"]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o.sum(axis=1), gold["o_sum"], rtol=1e-12, atol=1e-12)
