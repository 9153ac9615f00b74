"""The allocation-free entry point (mla_decode_noalloc) against mla_decode through the C
ABI: the same plan and inputs must give the same bits, on two calls in a row with the
second one smaller (the scratch array keeps the first call's contents), and plans larger
than the scratch array are refused before anything runs."""
import numpy as np
import pytest
import torch

from decode_attention_gather_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    from decode_attention_gather_amd import mla as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def _both(mla, case, split):
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads, split_kv=split)
    o_ref, lse_ref = mla.run_decode(dc, plan)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    mla.decode_noalloc(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
                       dc.output_scale, o, lse)
    torch.cuda.synchronize()
    return o, lse, o_ref, lse_ref


@pytest.mark.parametrize("first,second", [
    (([131072] * 4, 12, 1, 0), ([700, 33], 12, 2, 3)),        # narrow kernel, then smaller
    (([4096, 20000], 12, 8, 0), ([3000], 12, 8, 4)),           # wide kernel, then smaller
    (([131072] * 2, 12, 1, 2), ([20000], 12, 1, 1)),           # shared splits (and the fold)
], ids=["narrow", "wide", "shared"])
def test_noalloc_matches_decode(mla, first, second):
    for i, (lens, heads, q_len, split) in enumerate((first, second)):
        print(f"[gpu] noalloc call {i}: lens={lens} H={heads} q={q_len} split={split}",
              flush=True)
        case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=300 + i)
        o, lse, o_ref, lse_ref = _both(mla, case, split)
        assert torch.equal(o, o_ref), "O differs from mla_decode"
        assert torch.equal(lse, lse_ref), "LSE differs from mla_decode"


def test_noalloc_refuses_large_plans(mla):
    case = inputs.make_case([64], num_heads=12, q_len=1, seed=5)
    dc = mla.to_device(case)
    o = torch.empty((12, 512), dtype=torch.bfloat16, device="cuda")
    # 4096 rows x 1024 splits of (512 + 4) fp32 values: far above 64 MiB
    big = mla.Plan([1 << 20] * 4, q_len=8, num_heads=128, split_kv=1024, max_split_kv=1024)
    assert big.workspace_size() > mla.NOALLOC_SCRATCH_BYTES
    with pytest.raises(mla.MlaError) as ei:
        mla.decode_noalloc(big, dc.q, dc.kv, dc.block_table, dc.kv_lens, 0.07, 1.0, o)
    assert ei.value.status == mla.MLA_ERR_WORKSPACE
    g = mla.Plan.graph(1, q_len=1, num_heads=12, max_kv_len=64)
    with pytest.raises(mla.MlaError) as ei:
        mla.decode_noalloc(g, dc.q, dc.kv, dc.block_table, dc.kv_lens, 0.07, 1.0, o)
    assert ei.value.status == mla.MLA_ERR_INVALID_ARG
