"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on seeded inputs.

Bar (element by element):
  |O_gpu - O_ref| <= 1e-2 + 1e-2 * |O_ref|        (BF16 output)
  |LSE_gpu - LSE_ref| <= 1e-4 * max(1, |LSE_ref|) (fp32 LSE; relative, with an absolute
                                                   floor where LSE is near 0)
Small cases are checked on every row; the full-size workloads, in the launch
configuration the benchmark times, on sampled rows the oracle computes one by one.
Inputs carry NaN poison in every cache byte the kernel must not read (see inputs.py),
so an out-of-range read shows up as a NaN mismatch.
"""
import math
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from decode_attention_gather_amd import inputs

pytestmark = pytest.mark.gpu

F32 = lambda x: float(np.float32(x))


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    from decode_attention_gather_amd import mla as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def run_gpu(mla, case, split_kv=None, max_split_kv=256, f32_out=False, dc=None):
    dc = dc or mla.to_device(case)
    sk = case.split_kv if split_kv is None else split_kv
    plan = mla.Plan(dc.kv_lens_host, q_len=case.q_len, num_heads=case.num_heads, split_kv=sk,
                    max_split_kv=max_split_kv)
    o, lse = mla.run_decode(dc, plan, f32_out=f32_out)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), plan


def run_oracle(case, rows=None):
    return oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=case.q_len,
                             num_heads=case.num_heads, softmax_scale=F32(case.softmax_scale),
                             output_scale=F32(case.output_scale), rows=rows)


def assert_parity(o, lse, o_ref, lse_ref, tag=""):
    assert np.isfinite(o).all(), f"{tag}: non-finite O"
    assert np.isfinite(lse).all(), f"{tag}: non-finite LSE"
    err = np.abs(o - o_ref)
    bound = 1e-2 + 1e-2 * np.abs(o_ref)
    worst = float((err / bound).max())
    lerr = np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    _say(f"  {tag}: worst |dO|/bound = {worst:.3f}, max |dLSE| rel = {float(lerr.max()):.2e}")
    assert (err <= bound).all(), f"{tag}: O mismatch, worst ratio {worst}"
    assert (lerr <= 1e-4).all(), f"{tag}: LSE mismatch {float(lerr.max())}"


SMALL = [
    # name, kv_lens, heads, q_len, split_kv
    ("q1_ragged_split3", [1, 100, 2049], 12, 1, 3),
    ("q8_causal_6tiles", [8, 777], 12, 8, 4),
    ("q3_h5_rows15", [33, 64, 3], 5, 3, 2),
    ("q8_last_split_one_token", [65, 97], 12, 8, 3),
    ("q1_single_split_long", [5000], 12, 1, 1),
    ("q2_h16_planner", [1500, 40, 2], 16, 2, 0),
    ("h96_q8_planner", [300, 1000], 96, 8, 0),
    ("q1_many_requests", [37 * i + 5 for i in range(1, 20)], 12, 1, 0),
    ("q4_h1_split5", [640, 641], 1, 4, 5),
    ("odd_pages_split2", [3 * 32 + 7, 5 * 32], 12, 1, 2),
    # row blocks of the wide kernel: 4 tiles (33-64 rows), 6 tiles with padding rows
    ("q4_h16_rows64", [500, 1234], 16, 4, 3),
    ("q4_h12_rows48_planner", [77, 2000], 12, 4, 0),
    ("q7_h12_rows84", [300, 900], 12, 7, 2),
    ("q8_h16_two_blocks", [64, 4000], 16, 8, 0),
]


def test_planner_cap_128(mla):
    """The pages' per-request cap of 128 splits (issue #20510, Repro 2), beside the
    default 256: a long request hits the cap, parity holds."""
    case = inputs.make_case([300000, 2000], num_heads=12, q_len=1, seed=77, split_kv=0)
    _say("[gpu] planner with max_split_kv=128")
    o, lse, plan = run_gpu(mla, case, max_split_kv=128)
    # 9375 pages in whole-page splits of at most 128: ceil(9375 / 74) = 127 splits
    assert plan.info()[1][0] == 127
    assert mla.Plan([300000, 2000], q_len=1, num_heads=12).info()[1][0] > 128
    rows = inputs.sample_rows(case, 24)
    o_ref, lse_ref = run_oracle(case, rows)
    assert_parity(o[rows], lse[rows], o_ref, lse_ref, "cap128")


@pytest.mark.parametrize("name,lens,heads,q_len,split", SMALL, ids=[s[0] for s in SMALL])
def test_small_parity(mla, name, lens, heads, q_len, split):
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=zlib.crc32(name.encode()) % 10000,
                            split_kv=split)
    _say(f"[gpu] small {name}: lens={lens} H={heads} q={q_len} split={split}")
    o, lse, _ = run_gpu(mla, case)
    o_ref, lse_ref = run_oracle(case)
    assert_parity(o, lse, o_ref, lse_ref, name)


def test_output_scale_and_extreme_scores(mla):
    case = inputs.make_case([300, 129], num_heads=12, q_len=2, seed=5, split_kv=3,
                            softmax_scale=0.5, output_scale=0.37)
    _say("[gpu] output_scale 0.37, softmax_scale 0.5")
    o, lse, _ = run_gpu(mla, case)
    o_ref, lse_ref = run_oracle(case)
    assert_parity(o, lse, o_ref, lse_ref, "scales")


@pytest.mark.parametrize("heads", [12, 48, 96])
def test_kv_len_one_and_equal_scores(mla, heads):
    # one key per request: O is that key's V (exactly representable in BF16)
    case = inputs.make_case([1, 1, 1], num_heads=heads, q_len=1, seed=6, split_kv=1)
    _say(f"[gpu] kv_len 1 H={heads}")
    o, lse, _ = run_gpu(mla, case)
    o_ref, lse_ref = run_oracle(case)
    assert np.array_equal(o, o_ref.astype(np.float32)), "kv_len 1 must return V exactly"
    assert_parity(o, lse, o_ref, lse_ref, "kv_len1")
    # q = 0: equal scores, O = mean of V
    case = inputs.make_case([100, 1000], num_heads=heads, q_len=1, seed=7, split_kv=4)
    case.q.zero_()
    _say(f"[gpu] equal scores H={heads}")
    o, lse, _ = run_gpu(mla, case)
    o_ref, lse_ref = run_oracle(case)
    assert_parity(o, lse, o_ref, lse_ref, "equal")
    np.testing.assert_allclose(lse, np.log([100.0] * heads + [1000.0] * heads), rtol=1e-6)


@pytest.mark.parametrize("lens,heads,q_len", [
    ([3000, 20000, 777], 12, 8),      # wide kernel, 96-row blocks
    ([131072, 3000, 777], 12, 1),     # narrow kernel, one row tile (the headline's)
    ([131072, 3000, 777], 16, 2),     # narrow kernel, two row tiles
    ([131072, 3000, 777], 12, 2),     # narrow kernel, two row tiles with padding rows
], ids=["wide_h12_q8", "narrow_h12_q1", "narrow_h16_q2", "narrow_h12_q2"])
def test_split_invariance_f32(mla, lens, heads, q_len):
    """fp32 O (before the BF16 cast) from different split plans agrees to 1e-5. Lengths
    3000 and 777 end inside a page and inside a two-page step, 131072 is the headline's."""
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=8)
    dc = mla.to_device(case)
    outs = []
    for sk in (1, 2, 5, 0, 13):
        _say(f"[gpu] split invariance H={heads} q={q_len} split_kv={sk}")
        o, lse, plan = run_gpu(mla, case, split_kv=sk, f32_out=True, dc=dc)
        outs.append((sk, o, lse))
    base = outs[0]
    for sk, o, lse in outs[1:]:
        d = float(np.abs(o - base[1]).max())
        dl = float(np.abs(lse - base[2]).max())
        _say(f"  split {sk} vs 1: max |dO| = {d:.3e}, max |dLSE| = {dl:.3e}")
        assert d <= 1e-5, (sk, d)
        assert dl <= 1e-5 * max(1.0, float(np.abs(base[2]).max())), (sk, dl)


@pytest.mark.parametrize("heads,q_len", [(12, 8), (16, 4), (96, 8), (12, 1)])
def test_large_score_range(mla, heads, q_len):
    """Scores spread over hundreds of log2 units (softmax_scale 4): within a split the
    running maximum jumps by far more than 2^64 between pages, and the weights of most
    earlier pages underflow to zero once rescaled."""
    case = inputs.make_case([5000, 700], num_heads=heads, q_len=q_len, seed=31, split_kv=2,
                            softmax_scale=4.0)
    _say(f"[gpu] large score range H={heads} q={q_len}")
    o, lse, _ = run_gpu(mla, case)
    o_ref, lse_ref = run_oracle(case)
    assert_parity(o, lse, o_ref, lse_ref, "large range")


@pytest.mark.parametrize("heads,q_len", [(12, 8), (12, 4), (16, 4), (12, 1), (96, 8)])
def test_determinism(mla, heads, q_len):
    """Repeated calls give the same bits (wide blocks of 6 and 4 row tiles, narrow)."""
    case = inputs.make_case([4096, 777], num_heads=heads, q_len=q_len, seed=9, split_kv=3)
    dc = mla.to_device(case)
    _say(f"[gpu] determinism H={heads} q={q_len}")
    o1, l1, _ = run_gpu(mla, case, dc=dc)
    for _ in range(2):
        o2, l2, _ = run_gpu(mla, case, dc=dc)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("lens,split,bounded,dt", [
    ([1, 100, 2049], 3, False, "e4m3"),          # ragged, steps % 3 of 0, 1 and 2
    ([5000], 2, False, "e4m3"),
    ([3 * 32 + 7, 5 * 32, 33], 2, True, "e4m3"),  # key windows inside pages
    ([131072], 6, False, "e4m3"),
    ([1, 100, 2049], 3, False, "bf16"),
    ([3 * 32 + 7, 5 * 32, 33], 2, True, "bf16"),
])
def test_loader_depth_same_bits(mla, lens, split, bounded, dt):
    """The one-tile kernels run another schedule when the grid has fewer work items than
    CUs (E4M3: three steps of loads in flight per loader instead of two; both: the
    waves' roles placed so that the QK SIMDs carry loaders): the partials (workspace)
    must be the same bits either way. num_cus 1 makes every grid full; 2 items - 1 CUs
    leaves the grid under-filled while every split still runs on one workgroup."""
    case = inputs.make_case(lens, num_heads=12, q_len=1, seed=41, split_kv=split, kv_dtype=dt)
    dc = mla.to_device(case)
    kvb = None
    if bounded:
        kvb = torch.tensor([[min(5, n), n] for n in lens], dtype=torch.int32, device="cuda")
    _say(f"[gpu] under-filled schedule lens={lens} split={split} bounded={bounded} {dt}")
    items = mla.Plan(dc.kv_lens_host, q_len=1, num_heads=12, split_kv=split, num_cus=1,
                     kv_dtype=dt).info()[0].work_items
    assert items >= 2
    ws = []
    for cus in (2 * items - 1, 1):
        plan = mla.Plan(dc.kv_lens_host, q_len=1, num_heads=12, split_kv=split, num_cus=cus,
                        kv_dtype=dt)
        assert plan.info()[0].split_workgroups == 1
        w = torch.zeros(plan.workspace_size(), dtype=torch.uint8, device="cuda")
        mla.partial_ex(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, case.softmax_scale, w,
                       kv_bounds=kvb)
        torch.cuda.synchronize()
        ws.append(w.cpu().numpy())
    assert ws[0].shape == ws[1].shape
    assert np.array_equal(ws[0], ws[1])


def test_device_lengths_shorter_than_plan(mla):
    """A device kv_len below the planned one leaves trailing splits empty; the result is
    the one for the shorter length."""
    case = inputs.make_case([640], num_heads=12, q_len=1, seed=10, split_kv=5)
    dc = mla.to_device(case)
    plan = mla.Plan([640], q_len=1, num_heads=12, split_kv=5)  # 5 splits of 4 pages
    dc.kv_lens.fill_(200)  # splits 2..4 become empty
    _say("[gpu] device lengths shorter than plan")
    o, lse = mla.run_decode(dc, plan)
    torch.cuda.synchronize()
    short = inputs.Case(q=case.q, kv=case.kv, block_table=case.block_table,
                        kv_lens=torch.tensor([200], dtype=torch.int32), q_len=1, num_heads=12)
    o_ref, lse_ref = run_oracle(short)
    assert_parity(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "short-device")


@pytest.mark.parametrize("lens,heads,q_len,split", [
    ([200000], 12, 1, 200),        # 8 dim slices per row (one long request)
    ([131072, 131072], 12, 8, 32),  # wide kernel partials, one slice
    ([40000, 300, 9000], 12, 2, 0),  # planner, uneven split counts
], ids=["slices8_q1", "wide_q8_split32", "planner_q2"])
def test_merge_width_sweep(mla, lens, heads, q_len, split):
    """PR #20380 (Test Coverage): the same partials merged with KvSplit 2/4/8/16 agree with
    KvSplit 1. Here: elementwise on the fp32 O and on LSE, to 1e-5."""
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=21)
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=q_len, num_heads=heads, split_kv=split)
    ws = plan.alloc_workspace()
    mla.partial(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale, ws)
    rows = case.rows
    outs = {}
    for gmax in (1, 2, 4, 8, 16):
        p = plan.with_merge_bound(gmax)
        g = p.info()[0].merge_groups
        o = torch.empty((rows, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
        mla.merge(p, ws, dc.output_scale, o, lse)
        torch.cuda.synchronize()
        outs[gmax] = (g, o.cpu().numpy(), lse.cpu().numpy())
        _say(f"[gpu] merge width bound {gmax}: groups {g}, slices {p.info()[0].merge_slices}")
    assert outs[16][0] >= 8, "the sweep must reach wide merges"
    _, o1, l1 = outs[1]
    assert np.isfinite(o1).all() and np.isfinite(l1).all()
    for gmax in (2, 4, 8, 16):
        _, o, lse = outs[gmax]
        d = float(np.abs(o - o1).max())
        dl = float((np.abs(lse - l1) / np.maximum(1.0, np.abs(l1))).max())
        _say(f"  KvSplit {gmax} vs 1: max |dO| = {d:.2e}, max |dLSE| rel = {dl:.2e}")
        assert d <= 1e-5 and dl <= 1e-5, (gmax, d, dl)
    o_ref, lse_ref = run_oracle(case, inputs.sample_rows(case, 12))
    assert_parity(o1[inputs.sample_rows(case, 12)], l1[inputs.sample_rows(case, 12)], o_ref,
                  lse_ref, "width sweep vs oracle")


# ---- merge kernel alone, on synthetic partials -------------------------------------

def _merge_reference(m, l, lt, O, S_list, out_scale):
    """fp64 combine of (m, l, l~, O) partials [parts, rows, ...] per request."""
    rows = m.shape[1]
    outs, lses = [], []
    base = 0
    for S in S_list:
        mm = m[base:base + S].astype(np.float64)
        M = np.max(mm, axis=0)
        w = np.where(np.isneginf(mm), 0.0, np.exp2(mm - M))
        Ls = (w * l[base:base + S]).sum(0)
        Lt = (w * lt[base:base + S]).sum(0)
        Osum = (w[:, :, None] * O[base:base + S]).sum(0)
        outs.append(out_scale * Osum / Lt[:, None])
        lses.append(math.log(2.0) * (M - 8.0 + np.log2(Ls)))
        base += S
    return np.concatenate(outs), np.concatenate(lses)


@pytest.mark.parametrize("lens,split,heads,q_len", [([1048576], 100, 12, 1), ([2048], 4, 12, 1),
                                                    ([131072] * 4, 25, 12, 1), ([5000, 90], 7, 3, 2)])
def test_merge_synthetic(mla, lens, split, heads, q_len):
    plan = mla.Plan(lens, q_len=q_len, num_heads=heads, split_kv=split)
    info, splits, _ = plan.info()
    rows = info.rows_per_request
    parts = info.total_splits
    g = torch.Generator().manual_seed(123)
    m = torch.randint(-20, 21, (parts, rows), generator=g).double().numpy()
    empty = torch.rand((parts, rows), generator=g).numpy() < 0.15
    m[empty] = -np.inf
    l = (torch.rand((parts, rows), generator=g).double().numpy() * 300.0 + 1.0)
    lt = l * (1.0 + 1e-3 * torch.randn((parts, rows), generator=g).double().numpy())
    O = torch.randn((parts, rows, 512), generator=g).double().numpy() * l[:, :, None] * 0.1
    l[empty] = 0.0
    lt[empty] = 0.0
    O[empty] = 0.0
    base = 0
    for S in splits:  # force one live partial per row of each request
        m[base, :] = np.where(np.isneginf(m[base, :]), 3.0, m[base, :])
        l[base, :] = np.where(l[base, :] == 0.0, 5.0, l[base, :])
        lt[base, :] = np.where(lt[base, :] == 0.0, 5.0, lt[base, :])
        base += S
    ws = plan.alloc_workspace()
    o_bytes = parts * rows * 512 * 4
    ws_o = ws[:o_bytes].view(torch.float32)
    ws_st = ws[o_bytes:o_bytes + parts * rows * 16].view(torch.float32)
    ws_o.copy_(torch.from_numpy(O.astype(np.float32).reshape(-1)))
    st = np.stack([m, l, lt, np.zeros_like(l)], axis=-1).astype(np.float32)
    ws_st.copy_(torch.from_numpy(st.reshape(-1)))
    # the reference takes the same fp32 values the kernel sees
    O32 = O.astype(np.float32).astype(np.float64)
    ref_o, ref_lse = _merge_reference(st[..., 0], st[..., 1].astype(np.float64),
                                      st[..., 2].astype(np.float64), O32, splits, 0.5)
    o = torch.empty((len(lens) * rows, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((len(lens) * rows,), dtype=torch.float32, device="cuda")
    _say(f"[gpu] merge synthetic lens={lens} split={split} groups={info.merge_groups}")
    mla.merge(plan, ws, 0.5, o, lse)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o.cpu().numpy(), ref_o, rtol=2e-5, atol=1e-6)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-5)
    ob = torch.empty((len(lens) * rows, 512), dtype=torch.bfloat16, device="cuda")
    mla.merge(plan, ws, 0.5, ob, None)
    torch.cuda.synchronize()
    # BF16 output is the RNE rounding of the fp32 result
    assert torch.equal(ob.cpu(), o.cpu().to(torch.bfloat16))


# ---- full-size workloads (launch configuration of the benchmark), sampled rows --------

FULL = ["c1_b1_h12_q1_2k", "c2_b4_h12_q1_128k", "c3_b16_h12_q8_128k", "c4_b1_h12_q1_1m",
        "c5_b8_h96_q8_mixed", "m_b16_h12_q1_128k", "s_b8_h12_q8_skewed", "t_b16_h16_q2_128k"]


@pytest.mark.parametrize("name", FULL)
def test_full_config_sampled(mla, name):
    _say(f"[gpu] full config {name}: generating inputs")
    case = inputs.make_config(name)
    rows = inputs.sample_rows_per_tile(case, 24)  # every row block of every request
    dc = mla.to_device(case)
    for sk in ([case.split_kv, 0] if case.split_kv else [0]):
        # the benchmark's plans (split cap 256)
        _say(f"[gpu] full config {name}: split_kv={sk}, {len(rows)} sampled rows")
        o, lse, plan = run_gpu(mla, case, split_kv=sk, max_split_kv=256, dc=dc)
        assert np.isfinite(o).all() and np.isfinite(lse).all()
        o_ref, lse_ref = run_oracle(case, rows)
        assert_parity(o[rows], lse[rows], o_ref, lse_ref, f"{name} split={sk}")
    del dc
    torch.cuda.empty_cache()
