"""Key windows (kv_bounds) through the C ABI against the fp64 oracle's windows.

Reading (issue #20510 "CuTe DSL FP8 MLA decode slower after #19338", Repro 1, where
kv_bounds is listed without a description): per request a half-open window
[start, end) of key positions, applied with the causal rule. Everything outside the
windows is poisoned: block-table entries of pages wholly outside point at the NaN page,
and the slots of each window's first and last page outside it hold NaN codes, so any
read of a key the method must not read shows up as a NaN mismatch.
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


def poisoned(case, bounds):
    """A copy of the case whose cache and block table hold NaN outside every window."""
    kv = case.kv.clone()
    bt = case.block_table.clone()
    nan_page = kv.shape[0] - 1
    nan = inputs.BF16_NAN if case.kv_dtype == "bf16" else inputs.E4M3_NAN
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        lo, hi = max(0, int(bounds[b, 0])), min(int(bounds[b, 1]), L)
        npg = (L + 31) // 32
        if hi <= lo:
            bt[b, :npg] = nan_page
            continue
        for p in range(npg):
            if 32 * (p + 1) <= lo or 32 * p >= hi:
                bt[b, p] = nan_page
        if lo % 32:
            kv[int(bt[b, lo // 32]), : lo % 32] = nan
        if hi % 32:
            kv[int(bt[b, (hi - 1) // 32]), hi % 32:] = nan
    return inputs.Case(q=case.q, kv=kv, block_table=bt, kv_lens=case.kv_lens, q_len=case.q_len,
                       num_heads=case.num_heads, softmax_scale=case.softmax_scale,
                       output_scale=case.output_scale, split_kv=case.split_kv,
                       kv_dtype=case.kv_dtype)


def oracle_bounded(case, bounds, sinks=None):
    return oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=case.q_len,
                             num_heads=case.num_heads, softmax_scale=F32(case.softmax_scale),
                             output_scale=F32(case.output_scale), kv_dtype=case.kv_dtype,
                             kv_bounds=bounds, sinks=sinks)


def assert_bounded(o, lse, o_ref, lse_ref, tag):
    """Parity where rows see keys; O = 0 and LSE = -inf exactly where a row sees none."""
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{tag}: rows without keys differ"
    assert (o[empty] == 0).all(), f"{tag}: O of rows without keys"
    live = ~empty
    assert_parity(o[live], lse[live], o_ref[live], lse_ref[live], tag)


def run_bounded(mla, case, bounds, split, sinks=None):
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads, split_kv=split,
                    kv_dtype=case.kv_dtype)
    kb = torch.from_numpy(np.ascontiguousarray(bounds, np.int32)).cuda()
    sk = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    o = torch.empty((case.rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.rows,), dtype=torch.float32, device="cuda")
    ws = plan.alloc_workspace()
    mla.decode_bounded(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, kb, dc.softmax_scale,
                       dc.output_scale, ws, o, lse, sinks=sk)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), dc, plan, kb


# lengths, windows: page-unaligned starts and ends, a window across split boundaries, one
# from a negative start, one past L, a whole request, an empty one, one inside one page
LENS = [1000, 300, 2049, 97, 640]
BOUNDS = np.array([[300, 707], [-5, 500], [37, 2049], [70, 70], [5, 29]], np.int32)

CASES = [
    # name, heads, q_len, split_kv, kv dtype (kernel family)
    ("fp8_narrow_h12_q1", 12, 1, 3, "e4m3"),
    ("fp8_narrow_h16_q2", 16, 2, 0, "e4m3"),
    ("fp8_wide_h12_q8", 12, 8, 4, "e4m3"),
    ("fp8_wide_h96_q8", 96, 8, 0, "e4m3"),
    ("bf16_narrow_h12_q1", 12, 1, 3, "bf16"),
    ("bf16_wide_h12_q8", 12, 8, 0, "bf16"),
]


@pytest.mark.parametrize("name,heads,q_len,split,dt", CASES, ids=[c[0] for c in CASES])
def test_bounds_parity(mla, name, heads, q_len, split, dt):
    case = poisoned(inputs.make_case(LENS, num_heads=heads, q_len=q_len, seed=611, split_kv=split,
                                     kv_dtype=dt), BOUNDS)
    _say(f"[gpu] kv_bounds {name}: lens={LENS} split={split}")
    o, lse, _, _, _ = run_bounded(mla, case, BOUNDS, split)
    o_ref, lse_ref = oracle_bounded(case, BOUNDS)
    assert_bounded(o, lse, o_ref, lse_ref, name)


def test_bounds_whole_window_is_plain(mla):
    case = inputs.make_case([1000, 77], num_heads=12, q_len=2, seed=612, split_kv=3)
    full = np.array([[0, 1000], [-3, 1 << 30]], np.int32)
    _say("[gpu] kv_bounds covering every key vs the plain call")
    o, lse, dc, plan, _ = run_bounded(mla, case, full, 3)
    o_p, lse_p = mla.run_decode(dc, plan)
    torch.cuda.synchronize()
    assert np.array_equal(o, o_p.float().cpu().numpy()) and np.array_equal(lse, lse_p.cpu().numpy())


def test_bounds_sinks_and_empty(mla):
    case = inputs.make_case([500, 300], num_heads=12, q_len=1, seed=613, split_kv=2)
    bounds = np.array([[100, 100], [10, 250]], np.int32)
    sinks = np.linspace(-3.0, 6.0, 12).astype(np.float32)
    _say("[gpu] kv_bounds with sinks and an empty window")
    o, lse, _, _, _ = run_bounded(mla, case, bounds, 2, sinks=sinks)
    o_ref, lse_ref = oracle_bounded(case, bounds, sinks=sinks.astype(np.float64))
    assert (o[:12] == 0).all()
    np.testing.assert_allclose(lse[:12], sinks, rtol=1e-6, atol=1e-6)
    assert_parity(o[12:], lse[12:], o_ref[12:], lse_ref[12:], "sinks+bounds")


@pytest.mark.parametrize("heads,q_len", [(12, 1), (12, 8)], ids=["narrow", "wide"])
def test_bounds_split_invariance_f32(mla, heads, q_len):
    """fp32 O from different split plans agrees to 1e-5 under the same windows."""
    case = poisoned(inputs.make_case([20000, 3000], num_heads=heads, q_len=q_len, seed=614),
                    np.array([[1234, 17777], [100, 2990]], np.int32))
    bounds = torch.tensor([[1234, 17777], [100, 2990]], dtype=torch.int32, device="cuda")
    dc = mla.to_device(case)
    outs = []
    for sk in (1, 3, 0, 17):
        plan = mla.Plan(dc.kv_lens_host, q_len=q_len, num_heads=heads, split_kv=sk)
        ws = plan.alloc_workspace()
        mla.partial_ex(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, ws,
                       kv_bounds=bounds)
        o = torch.empty((case.rows, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((case.rows,), dtype=torch.float32, device="cuda")
        mla.merge(plan, ws, dc.output_scale, o, lse)
        torch.cuda.synchronize()
        outs.append((sk, o.cpu().numpy(), lse.cpu().numpy()))
        _say(f"[gpu] bounded split invariance H={heads} q={q_len} split_kv={sk}")
    for sk, o, lse in outs[1:]:
        d = float(np.abs(o - outs[0][1]).max())
        dl = float(np.abs(lse - outs[0][2]).max())
        _say(f"  split {sk} vs 1: max |dO| = {d:.2e}, max |dLSE| = {dl:.2e}")
        assert d <= 1e-5 and dl <= 1e-5 * max(1.0, float(np.abs(outs[0][2]).max()))
    o_ref, lse_ref = oracle_bounded(case, bounds.cpu().numpy(), None)
    rows = inputs.sample_rows(case, 16)
    assert_parity(outs[0][1][rows], outs[0][2][rows], o_ref[rows], lse_ref[rows], "bounded f32")


@pytest.mark.parametrize("dt", ["e4m3", "bf16"])
def test_bounds_graph_equals_host(mla, dt):
    case = poisoned(inputs.make_case(LENS, num_heads=12, q_len=2, seed=615, kv_dtype=dt), BOUNDS)
    _say(f"[gpu] kv_bounds graph path vs host path ({dt})")
    o_h, lse_h, dc, _, kb = run_bounded(mla, case, BOUNDS, 0)
    gp = mla.Plan.graph(len(LENS), q_len=2, num_heads=12, max_kv_len=max(LENS), kv_dtype=dt)
    ws = gp.alloc_workspace()
    o = torch.empty((case.rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((case.rows,), dtype=torch.float32, device="cuda")
    ss = torch.tensor([dc.softmax_scale], dtype=torch.float32, device="cuda")
    os_ = torch.tensor([dc.output_scale], dtype=torch.float32, device="cuda")
    mla.decode_graph_bounded(gp, dc.q, dc.kv, dc.block_table, dc.kv_lens, kb, ss, os_, ws, o, lse)
    torch.cuda.synchronize()
    assert np.array_equal(o.float().cpu().numpy(), o_h) and np.array_equal(lse.cpu().numpy(), lse_h)
    o_ref, lse_ref = oracle_bounded(case, BOUNDS)
    assert_bounded(o_h, lse_h, o_ref, lse_ref, f"graph bounds {dt}")
