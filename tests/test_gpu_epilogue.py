"""Merge epilogue variants through the C ABI: attention sinks and the MXFP8 form of O.

Checks:
  * sinks: parity with the fp64 oracle's sink definition (same bar as the plain path),
    sinks of -inf reproduce the plain call bit for bit, a sink far above every score;
  * MXFP8 on synthetic partials chosen so that the merged values are exact in fp32:
    BF16 O, E4M3 codes and E8M0 scales equal the oracle's rounding and quantization
    bit for bit (ties, block-scale boundaries, signed zeros, BF16 subnormals);
  * MXFP8 on real decode batches: the BF16 O next to it is the plain call's, the
    dequantized MXFP8 values meet the parity bar widened by one E4M3 rounding, and the
    codes and scales are the quantization of the BF16 O written beside them;
  * the graph path with both options equals the host-planned call, and a request of
    length 0 gives O = 0 with LSE = its head's sink; sinks changed between replays of a
    captured call take effect.
"""
import math

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


def oracle_rows(case, sinks=None, rows=None):
    return oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=case.q_len,
                             num_heads=case.num_heads, softmax_scale=F32(case.softmax_scale),
                             output_scale=F32(case.output_scale), rows=rows, sinks=sinks)


def make_sinks(case, seed, extra=()):
    """fp32 sink logits per head around the rows' typical LSE, plus fixed values."""
    g = np.random.default_rng(seed)
    H = case.num_heads
    ln_l = math.log(max(1, int(case.kv_lens.float().mean())))
    s = (ln_l + g.uniform(-2.0, 4.0, size=H)).astype(np.float32)
    for i, v in enumerate(extra):
        s[i % H] = v
    return s


def run_ex(mla, dc, plan, rows, sinks=None, fp8=False, bf16=True, lse=True):
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda") if bf16 else None
    ls = torch.empty((rows,), dtype=torch.float32, device="cuda") if lse else None
    c = torch.empty((rows, 512), dtype=torch.uint8, device="cuda") if fp8 else None
    sc = torch.empty((rows, 16), dtype=torch.uint8, device="cuda") if fp8 else None
    sk = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    ws = plan.alloc_workspace()
    mla.decode_ex(plan, dc.q, dc.kv, dc.block_table, dc.kv_lens, dc.softmax_scale,
                  dc.output_scale, ws, o, ls, sinks=sk, o_fp8=c, o_fp8_scales=sc)
    torch.cuda.synchronize()
    return o, ls, c, sc


def np_of(t):
    return None if t is None else (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


SINK_CASES = [
    # name, kv_lens, heads, q_len, split_kv, fixed sink values
    ("h12_q1_split3", [1, 100, 2049], 12, 1, 3, (30.0, -np.inf, -5.0)),
    ("h12_q8_wide", [8, 777], 12, 8, 4, (1000.0, -np.inf)),
    ("h16_q2_planner", [1500, 40, 2], 16, 2, 0, (-np.inf, 12.0)),
    ("h96_q8_planner", [300, 1000], 96, 8, 0, (25.0,)),
]


@pytest.mark.parametrize("name,lens,heads,q_len,split,extra", SINK_CASES,
                         ids=[c[0] for c in SINK_CASES])
def test_sinks_parity(mla, name, lens, heads, q_len, split, extra):
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=515, split_kv=split)
    sinks = make_sinks(case, 7, extra)
    _say(f"[gpu] sinks {name}: lens={lens} H={heads} q={q_len} split={split}")
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=q_len, num_heads=heads, split_kv=split)
    o, lse, _, _ = run_ex(mla, dc, plan, case.rows, sinks=sinks)
    o_ref, lse_ref = oracle_rows(case, sinks=sinks.astype(np.float64))
    assert_parity(np_of(o), np_of(lse), o_ref, lse_ref, name)


def test_sinks_minus_inf_is_plain(mla):
    case = inputs.make_case([3000, 777], num_heads=12, q_len=8, seed=516, split_kv=3)
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=8, num_heads=12, split_kv=3)
    _say("[gpu] sinks of -inf vs the plain call")
    o, lse, _, _ = run_ex(mla, dc, plan, case.rows, sinks=np.full(12, -np.inf, np.float32))
    o_p, lse_p = mla.run_decode(dc, plan)
    torch.cuda.synchronize()
    assert torch.equal(o, o_p) and torch.equal(lse, lse_p)


# ---- MXFP8, bit-exact on synthetic partials ---------------------------------------------

def _target_rows(seed, nrows):
    """fp32 rows whose 32-element blocks cover the quantizer's edge cases."""
    g = np.random.default_rng(seed)
    rows = []
    for i in range(nrows):
        k = [-30, -8, -3, 0, 2, 5, 9, 14, 20][i % 9]
        x = g.standard_normal(512) * 2.0 ** k
        rows.append(x)
    x = rows[0]
    x[0:32] = 448.0
    x[32:64] = -448.0 * 2.0 ** -5
    x[64] = 448.0 * (1 + 2.0 ** -7)                # one BF16 step above 448: e goes up
    x[96] = 1.75                                   # exactly 448 * 2^-8: e goes up too
    x[128] = 1.875
    x[160:192] = 0.0
    x[192:224] = -0.0
    x[224:256] = np.ldexp(1.0 + np.arange(32) / 8.0, -3)   # E4M3 ties after scaling
    x[256:288] = np.ldexp(1.0 + np.arange(32) / 16.0, 7)   # more ties, other exponent
    rows[1][0:32] = np.ldexp(g.integers(1, 100, 32).astype(np.float64), -140)  # BF16 subnormals
    rows[1][32:64] = np.ldexp(1.0, -126) * (1 + np.arange(32) / 64.0)          # normal floor
    # the low end of the E8M0 range: amax = 448 * 2^-127 takes scale byte 1; one BF16
    # step below it, scale byte 0 and the block saturates (zeros stay zeros)
    rows[1][64:96] = 0.0
    rows[1][64], rows[1][65] = 1.75 * 2.0 ** -119, -2.0 ** -133
    rows[1][96:128] = 0.0
    rows[1][96], rows[1][97], rows[1][98] = 1.7421875 * 2.0 ** -119, -2.0 ** -125, -0.0
    return np.stack(rows).astype(np.float32)


def test_mxfp8_synthetic_exact(mla):
    lens, heads = [64, 64], 12
    plan = mla.Plan(lens, q_len=1, num_heads=heads, split_kv=1)
    info, splits, _ = plan.info()
    assert splits == [1, 1] and info.merge_groups == 1
    rows = len(lens) * heads
    target = _target_rows(91, rows)                       # the merged O, fp32-exact
    k = (np.arange(rows) % 8 + 1).astype(np.float64)      # l = l~ = 2^k per row
    ws = plan.alloc_workspace()
    o_bytes = rows * 512 * 4
    ws_o = ws[:o_bytes].view(torch.float32)
    ws_st = ws[o_bytes:o_bytes + rows * 16].view(torch.float32)
    ws_o.copy_(torch.from_numpy((target.astype(np.float64) * np.exp2(k)[:, None])
                                .astype(np.float32).reshape(-1)))
    st = np.stack([np.zeros(rows), np.exp2(k), np.exp2(k), np.zeros(rows)], -1).astype(np.float32)
    ws_st.copy_(torch.from_numpy(st.reshape(-1)))
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((rows, 512), dtype=torch.uint8, device="cuda")
    sc = torch.empty((rows, 16), dtype=torch.uint8, device="cuda")
    # the merge forms 0 + sum of weighted partials, times output_scale / l: a -0 partial
    # comes out as +0, and a negative output_scale flips every sign (zeros included)
    for out_scale in (1.0, -1.0):
        _say(f"[gpu] MXFP8 epilogue on synthetic partials (bit-exact), scale {out_scale}")
        mla.merge_ex(plan, ws, out_scale, o, None, o_fp8=c, o_fp8_scales=sc)
        torch.cuda.synchronize()
        merged = out_scale * (target.astype(np.float64) + 0.0)
        bf = oracle.round_bf16(merged)
        codes, scales = oracle.mxfp8_quantize(bf)
        got = np_of(o).astype(np.float64)
        bad = (got != bf) | (np.signbit(got) != np.signbit(bf))
        assert not bad.any(), np.argwhere(bad)[:5]
        assert np.array_equal(sc.cpu().numpy(), scales), \
            np.argwhere(sc.cpu().numpy() != scales)[:5]
        assert np.array_equal(c.cpu().numpy(), codes), np.argwhere(c.cpu().numpy() != codes)[:5]
        _check_mx_of_bf16(np_of(o), c.cpu().numpy(), sc.cpu().numpy())  # a second route
    # without the BF16 pointer the MXFP8 pair is unchanged
    c2 = torch.empty_like(c)
    sc2 = torch.empty_like(sc)
    mla.merge_ex(plan, ws, -1.0, None, None, o_fp8=c2, o_fp8_scales=sc2)
    torch.cuda.synchronize()
    assert torch.equal(c2, c) and torch.equal(sc2, sc)


# ---- MXFP8 on real batches ------------------------------------------------------------

def _check_mx_of_bf16(bf16, codes, scales):
    """The codes and scales are the MXFP8 quantization of the BF16 values beside them
    (PR #17441, commit messages on the quantize tile and its scale byte 0): the smallest
    power-of-two scale with amax < 448 * 2^e (strictly) per block, the RNE E4M3 cast
    (torch's) of x / 2^e, and +-448 for the non-zero values of a scale-byte-0 block."""
    xb = bf16.reshape(-1, 16, 32).astype(np.float64)
    e = scales.astype(np.int64).reshape(-1, 16) - 127
    amax = np.abs(xb).max(axis=2)
    assert (amax < 448.0 * np.ldexp(1.0, e)).all(), "scale too small"
    assert ((e == -127) | (amax >= 448.0 * np.ldexp(1.0, e - 1))).all(), "scale not minimal"
    y = (xb / np.ldexp(1.0, e)[:, :, None]).reshape(bf16.shape).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(xb.shape)
    sat = np.where(xb != 0, 0x7E, 0x00) | np.where(np.signbit(xb), 0x80, 0x00)
    ref = np.where((e == -127)[:, :, None], sat, ref).astype(np.uint8).reshape(codes.shape)
    assert np.array_equal(codes, ref), np.argwhere(codes != ref)[:5]


MX_CASES = [
    ("h12_q1_split3", [1, 100, 2049], 12, 1, 3),
    ("h12_q8_wide", [8, 777], 12, 8, 4),
    ("h96_q8_planner", [300, 1000], 96, 8, 0),
]


@pytest.mark.parametrize("name,lens,heads,q_len,split", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_mxfp8_decode(mla, name, lens, heads, q_len, split):
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=517, split_kv=split)
    dc = mla.to_device(case)
    plan = mla.Plan(dc.kv_lens_host, q_len=q_len, num_heads=heads, split_kv=split)
    _say(f"[gpu] MXFP8 decode {name}")
    o, lse, c, sc = run_ex(mla, dc, plan, case.rows, fp8=True)
    o_p, lse_p = mla.run_decode(dc, plan)
    torch.cuda.synchronize()
    assert torch.equal(o, o_p) and torch.equal(lse, lse_p), "BF16 O / LSE differ from plain"
    bf = np_of(o)
    codes, scales = c.cpu().numpy(), sc.cpu().numpy()
    _check_mx_of_bf16(bf, codes, scales)
    o_ref, lse_ref = oracle_rows(case)
    e = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    tab = oracle.e4m3_table()
    deq = tab[codes] * np.ldexp(1.0, e)
    base = 1e-2 + 1e-2 * np.abs(o_ref)
    bound = base * (1 + 2.0 ** -4) + 2.0 ** -4 * np.abs(o_ref) + np.ldexp(1.0, e - 10)
    worst = float((np.abs(deq - o_ref) / bound).max())
    _say(f"  {name}: MXFP8 worst |d|/bound = {worst:.3f}")
    assert (np.abs(deq - o_ref) <= bound).all()


# ---- graph path ------------------------------------------------------------------------

def test_epilogue_graph_equals_host(mla):
    lens, heads, q_len = [3000, 777, 64], 12, 2
    case = inputs.make_case(lens, num_heads=heads, q_len=q_len, seed=518, split_kv=0)
    dc = mla.to_device(case)
    sinks = make_sinks(case, 9, (40.0,))
    _say("[gpu] graph path with sinks and MXFP8 vs the host-planned call")
    hp = mla.Plan(dc.kv_lens_host, q_len=q_len, num_heads=heads, split_kv=0)
    o_h, lse_h, c_h, sc_h = run_ex(mla, dc, hp, case.rows, sinks=sinks, fp8=True)
    gp = mla.Plan.graph(len(lens), q_len=q_len, num_heads=heads, max_kv_len=max(lens))
    ws = gp.alloc_workspace()
    o = torch.empty_like(o_h)
    lse = torch.empty_like(lse_h)
    c = torch.empty_like(c_h)
    sc = torch.empty_like(sc_h)
    sk = torch.from_numpy(sinks).cuda()
    ss = torch.tensor([dc.softmax_scale], dtype=torch.float32, device="cuda")
    os_ = torch.tensor([dc.output_scale], dtype=torch.float32, device="cuda")
    mla.decode_graph_ex(gp, dc.q, dc.kv, dc.block_table, dc.kv_lens, ss, os_, ws, o, lse,
                        sinks=sk, o_fp8=c, o_fp8_scales=sc)
    torch.cuda.synchronize()
    assert torch.equal(o, o_h) and torch.equal(lse, lse_h)
    assert torch.equal(c, c_h) and torch.equal(sc, sc_h)
    o_ref, lse_ref = oracle_rows(case, sinks=sinks.astype(np.float64))
    assert_parity(np_of(o), np_of(lse), o_ref, lse_ref, "graph sinks")

    # a request of length 0: O = 0 and LSE = the head's sink
    lens0 = torch.tensor([0, 777, 64], dtype=torch.int32, device="cuda")
    mla.decode_graph_ex(gp, dc.q, dc.kv, dc.block_table, lens0, ss, os_, ws, o, lse,
                        sinks=sk, o_fp8=c, o_fp8_scales=sc)
    torch.cuda.synchronize()
    r0 = q_len * heads
    assert (np_of(o)[:r0] == 0).all() and (c.cpu().numpy()[:r0] & 0x7F == 0).all()
    sink_of_row = np.tile(sinks, q_len).astype(np.float64)
    np.testing.assert_allclose(np_of(lse)[:r0], sink_of_row, rtol=1e-6, atol=1e-6)


def test_epilogue_graph_replay_changes_sinks(mla):
    lens, heads = [2000, 500], 12
    case = inputs.make_case(lens, num_heads=heads, q_len=1, seed=519, split_kv=0)
    dc = mla.to_device(case)
    gp = mla.Plan.graph(2, q_len=1, num_heads=heads, max_kv_len=2000)
    ws = gp.alloc_workspace()
    rows = case.rows
    o = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows,), dtype=torch.float32, device="cuda")
    ss = torch.tensor([dc.softmax_scale], dtype=torch.float32, device="cuda")
    os_ = torch.tensor([1.0], dtype=torch.float32, device="cuda")
    sk = torch.zeros(heads, dtype=torch.float32, device="cuda")

    def call(stream=None):
        mla.decode_graph_ex(gp, dc.q, dc.kv, dc.block_table, dc.kv_lens, ss, os_, ws, o, lse,
                            sinks=sk, stream=stream)

    call()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
    torch.cuda.synchronize()
    for i, v in enumerate((-np.inf, 5.0, 20.0)):
        sinks = make_sinks(case, 100 + i, (v,))
        sk.copy_(torch.from_numpy(sinks))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[gpu] graph replay {i} with new sinks")
        o_ref, lse_ref = oracle_rows(case, sinks=sinks.astype(np.float64))
        assert_parity(np_of(o), np_of(lse), o_ref, lse_ref, f"replay {i}")
