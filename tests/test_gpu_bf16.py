"""The BF16 cache variant through the C ABI (plans built with kv_dtype "bf16").

Same bar as tests/test_gpu_parity.py against the fp64 oracle's BF16 path: every row of
small cases (several row blocks, ragged tails, causal q > 1, splits with empty causal
rows), sampled rows of the full-size BF16 workloads in the benchmark's launch
configuration, split-count invariance of the fp32 merge to 1e-5, the graph path equal
to the host-planned call bit for bit, and ragged query counts.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_gather_amd import inputs
from test_gpu_parity import F32, _say, assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    from decode_attention_gather_amd import mla as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def oracle_bf16(case, rows=None, q_lens=None):
    return oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=case.q_len,
                             num_heads=case.num_heads, softmax_scale=F32(case.softmax_scale),
                             output_scale=F32(case.output_scale), rows=rows, kv_dtype="bf16")


def run_bf16(mla, case, split_kv=None, dc=None, f32_out=False):
    dc = dc or mla.to_device(case)
    sk = case.split_kv if split_kv is None else split_kv
    plan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads, split_kv=sk,
                    kv_dtype="bf16")
    o, lse = mla.run_decode(dc, plan, f32_out=f32_out)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), plan


SMALL = [
    # name, kv_lens, heads, q_len, split_kv
    ("q1_ragged_split3", [1, 100, 2049], 12, 1, 3),
    ("q8_causal_three_blocks", [8, 777], 12, 8, 4),
    ("q3_h5_rows15", [33, 64, 3], 5, 3, 2),
    ("q2_h16_planner", [1500, 40, 2], 16, 2, 0),
    ("h96_q2_planner", [300, 1000], 96, 2, 0),
    ("q1_single_split_long", [5000], 12, 1, 1),
    ("odd_pages_split2", [3 * 32 + 7, 5 * 32], 12, 1, 2),
    ("q8_last_split_one_token", [65, 97], 12, 8, 3),
    # wide row blocks: ragged row counts inside a block, two blocks, two-page splits
    ("q7_h16_two_wide_blocks", [700, 33], 16, 7, 2),
    ("q13_h5_rows65", [400, 129], 5, 13, 0),
    ("q5_h16_rows80_split1", [1000], 16, 5, 1),
    ("q6_h16_two_pages", [64, 40], 16, 6, 1),
]


@pytest.mark.parametrize("name,lens,heads,q_len,split", SMALL, ids=[s[0] for s in SMALL])
def test_bf16_small_parity(mla, name, lens, heads, q_len, split):
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=9001, split_kv=split,
                            kv_dtype="bf16")
    _say(f"[gpu] bf16 {name}: lens={lens} H={heads} q={q_len} split={split}")
    o, lse, _ = run_bf16(mla, case)
    o_ref, lse_ref = oracle_bf16(case)
    assert_parity(o, lse, o_ref, lse_ref, name)


def test_bf16_single_key_and_equal_scores(mla):
    case = inputs.make_case([1, 40], num_heads=12, q_len=1, seed=9002, split_kv=0,
                            kv_dtype="bf16")
    case.q[1].zero_()  # request 1: equal scores, O = mean of V
    _say("[gpu] bf16 kv_len 1 and equal scores")
    o, lse, _ = run_bf16(mla, case)
    o_ref, lse_ref = oracle_bf16(case)
    assert_parity(o, lse, o_ref, lse_ref, "bf16 special cases")


@pytest.mark.parametrize("q_len", [2, 8])
def test_bf16_split_invariance_f32(mla, q_len):
    case = inputs.make_case([3000], num_heads=12, q_len=q_len, seed=9003, kv_dtype="bf16")
    dc = mla.to_device(case)
    outs = []
    for sk in (1, 3, 7, 0):
        _say(f"[gpu] bf16 split invariance q_len={q_len} split_kv={sk}")
        o, lse, _ = run_bf16(mla, case, split_kv=sk, dc=dc, f32_out=True)
        outs.append((o, lse))
    for o, lse in outs[1:]:
        np.testing.assert_allclose(o, outs[0][0], rtol=0, atol=1e-5)
        np.testing.assert_allclose(lse, outs[0][1], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("heads,q_len", [(12, 8), (12, 4), (16, 7), (12, 1)])
def test_bf16_determinism(mla, heads, q_len):
    """Repeated calls give the same bits (wide blocks of 6 and 4 row tiles, narrow)."""
    case = inputs.make_case([4096, 777], num_heads=heads, q_len=q_len, seed=19, split_kv=3,
                            kv_dtype="bf16")
    dc = mla.to_device(case)
    _say(f"[gpu] bf16 determinism H={heads} q={q_len}")
    o1, l1, _ = run_bf16(mla, case, dc=dc)
    for _ in range(2):
        o2, l2, _ = run_bf16(mla, case, dc=dc)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_bf16_graph_equals_host_and_varq(mla):
    lens = [3000, 777, 64]
    case = inputs.make_case(lens, num_heads=12, q_len=4, seed=9004, kv_dtype="bf16")
    dc = mla.to_device(case)
    _say("[gpu] bf16 graph path vs host plan")
    o_h, lse_h, _ = run_bf16(mla, case, split_kv=0, dc=dc)
    gp = mla.Plan.graph(3, q_len=4, num_heads=12, max_kv_len=3000, kv_dtype="bf16")
    ws = gp.alloc_workspace()
    o = torch.empty((case.rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.rows,), dtype=torch.float32, device="cuda")
    ss = torch.tensor([case.softmax_scale], dtype=torch.float32, device="cuda")
    os_ = torch.tensor([1.0], dtype=torch.float32, device="cuda")
    mla.decode_graph(gp, dc.q, dc.kv, dc.block_table, dc.kv_lens, ss, os_, ws, o, lse)
    torch.cuda.synchronize()
    assert np.array_equal(o.float().cpu().numpy(), o_h) and np.array_equal(lse.cpu().numpy(), lse_h)
    # ragged query counts: rows past q_lens[b] are O = 0, LSE = -inf; the others follow
    # the oracle on that request alone with its own count
    q_lens = [4, 1, 3]
    _say(f"[gpu] bf16 ragged q_lens={q_lens}")
    hp = mla.Plan(dc.kv_lens_host, q_len=4, num_heads=12, split_kv=0, kv_dtype="bf16")
    wsh = hp.alloc_workspace()
    mla.decode(hp, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, 1.0, wsh, o, lse,
               q_lens=torch.tensor(q_lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o_np, lse_np = o.float().cpu().numpy(), lse.cpu().numpy()
    H = 12
    for b, qb in enumerate(q_lens):
        sub = inputs.Case(q=case.q[b:b + 1, :qb].contiguous(), kv=case.kv,
                          block_table=case.block_table[b:b + 1].contiguous(),
                          kv_lens=case.kv_lens[b:b + 1].clone(), q_len=qb, num_heads=H,
                          softmax_scale=case.softmax_scale, kv_dtype="bf16")
        ob, lb = oracle_bf16(sub)
        r0 = b * 4 * H
        assert_parity(o_np[r0:r0 + qb * H], lse_np[r0:r0 + qb * H], ob, lb, f"varq b={b}")
        assert (o_np[r0 + qb * H:r0 + 4 * H] == 0).all()
        assert np.isneginf(lse_np[r0 + qb * H:r0 + 4 * H]).all()


FULL = ["b_b1_h12_q8_1m_bf16", "b_b16_h12_q1_128k_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_bf16_full_config_sampled(mla, name):
    _say(f"[gpu] bf16 full config {name}: generating inputs")
    case = inputs.make_config(name)
    rows = inputs.sample_rows(case, 24)
    dc = mla.to_device(case)
    for sk in ([case.split_kv, 0] if case.split_kv else [0]):
        _say(f"[gpu] bf16 full config {name}: split_kv={sk}")
        o, lse, _ = run_bf16(mla, case, split_kv=sk, dc=dc)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        o_ref, lse_ref = oracle_bf16(case, rows)
        assert_parity(o[rows], lse[rows], o_ref, lse_ref, f"{name} split={sk}")
    del dc
    torch.cuda.empty_cache()
