"""Checks that pin the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes ``lib_path`` (None = the real oracle) and raises
AssertionError when the oracle disagrees with:
  * torch's own float8_e4m3fn decoding (a separate library routine);
  * exact rational arithmetic (``fractions.Fraction``) for the score of a single key;
  * closed forms: one key gives O = V, equal scores give the mean of V and LSE = ln n;
  * 50-digit brute force (mpmath) with no max subtraction, on tiny inputs;
  * torch's fp64 scaled_dot_product_attention and logsumexp on the gathered rows;
  * invariances of the definition: permuting physical pages with the block table,
    re-expressing a row as a split-and-merge over page-aligned key ranges, and the
    causal rule that query j of an MTP step equals a q_len = 1 step over its prefix.

The definition being pinned (TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower
after #19338", Setup and Repro 1): 576-byte E4M3 rows (512 latent + 64 rope), V = the
latent, page size 32, scores softmax_scale * q.k, output_scale on O only, and for the
q = 8 MTP verify step query j attends to KV[0 .. L - 8 + j].
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

import oracle
from decode_attention_gather_amd import inputs

F32_SCALE = float(np.float32(inputs.SOFTMAX_SCALE))


def _run(case, lib_path, rows=None, **kw):
    return oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens,
                             q_len=case.q_len, num_heads=case.num_heads,
                             softmax_scale=kw.get("softmax_scale", F32_SCALE),
                             output_scale=kw.get("output_scale", case.output_scale),
                             rows=rows, lib_path=lib_path, sinks=kw.get("sinks"),
                             kv_dtype=case.kv_dtype)


def _gather(case, b, n):
    """Gather the first n cached rows of request b with torch indexing -> uint8 [n, 576]."""
    tok = torch.arange(n)
    pages = case.block_table[b].to(torch.int64)[tok // inputs.PAGE]
    return case.kv[pages, tok % inputs.PAGE]


def _dec(codes_u8: torch.Tensor) -> torch.Tensor:
    return codes_u8.view(torch.float8_e4m3fn).to(torch.float64)


def _dec_case(case, codes: torch.Tensor) -> torch.Tensor:
    """fp64 values of q or cache elements of a case, E4M3 or BF16, via torch."""
    if case.kv_dtype == "bf16":
        return codes.view(torch.bfloat16).to(torch.float64)
    return _dec(codes)


def pin_e4m3_table(lib_path=None):
    ours = oracle.e4m3_table(lib_path)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    nan_ours, nan_ref = np.isnan(ours), np.isnan(ref)
    assert (nan_ours == nan_ref).all(), "NaN codes differ"
    assert nan_ours.sum() == 2 and nan_ours[0x7F] and nan_ours[0xFF]
    assert np.array_equal(ours[~nan_ours], ref[~nan_ref]), "finite E4M3 values differ"
    assert np.array_equal(np.signbit(ours[~nan_ours]), np.signbit(ref[~nan_ref]))


def pin_single_key(lib_path=None):
    """kv_len 1: O = output_scale * V_0 exactly and LSE = s_0 (exact rational score)."""
    case = inputs.make_case([1, 1], num_heads=3, q_len=1, seed=11, output_scale=1.5)
    o, lse = _run(case, lib_path)
    tab = [Fraction(v) if not math.isnan(v) else None for v in
           torch.arange(256).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()]
    for b in range(case.batch):
        k = _gather(case, b, 1)[0]
        v = _dec(k[:inputs.D_V]).numpy()
        for h in range(case.num_heads):
            r = b * case.num_heads + h
            qrow = case.q[b, 0, h]
            dot = sum(tab[int(a)] * tab[int(c)] for a, c in zip(qrow.tolist(), k.tolist()))
            s0 = float(Fraction(F32_SCALE) * dot)
            assert lse[r] == s0, (lse[r], s0)
            assert np.array_equal(o[r], 1.5 * v), "O != output_scale * V_0"


def pin_equal_scores(lib_path=None):
    """q = 0 gives equal scores: O is the mean of the visible V rows, LSE = ln n."""
    case = inputs.make_case([37, 64, 5], num_heads=2, q_len=3, seed=12)
    case.q.zero_()
    o, lse = _run(case, lib_path)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        for j in range(case.q_len):
            n = L - case.q_len + j + 1
            mean = _dec(_gather(case, b, n)[:, :inputs.D_V]).mean(dim=0).numpy()
            for h in range(case.num_heads):
                r = (b * case.q_len + j) * case.num_heads + h
                np.testing.assert_allclose(o[r], mean, rtol=1e-13, atol=1e-13)
                assert abs(lse[r] - math.log(n)) <= 1e-14 * max(1.0, math.log(n))


def pin_mpmath_bruteforce(lib_path=None):
    """Tiny inputs against 50-digit arithmetic with no max subtraction."""
    import mpmath
    mpmath.mp.dps = 50
    case = inputs.make_case([3, 8, 2], num_heads=2, q_len=2, seed=13, output_scale=0.75)
    o, lse = _run(case, lib_path)
    sc = mpmath.mpf(F32_SCALE)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        for j in range(case.q_len):
            n = L - case.q_len + j + 1
            rows = _dec(_gather(case, b, n)).tolist()
            for h in range(case.num_heads):
                r = (b * case.q_len + j) * case.num_heads + h
                qv = _dec(case.q[b, j, h]).tolist()
                es = []
                for i in range(n):
                    dot = mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c) for a, c in zip(qv, rows[i]))
                    es.append(mpmath.exp(sc * dot))
                tot = mpmath.fsum(es)
                ref_lse = float(mpmath.log(tot))
                assert abs(lse[r] - ref_lse) <= 1e-13 * max(1.0, abs(ref_lse)), (lse[r], ref_lse)
                for d in range(0, inputs.D_V, 7):
                    ref = float(mpmath.mpf("0.75") *
                                mpmath.fsum(es[i] * rows[i][d] for i in range(n)) / tot)
                    assert abs(o[r, d] - ref) <= 1e-13 * max(1.0, abs(ref)), (d, o[r, d], ref)


def pin_sdpa(lib_path=None):
    """fp64 torch SDPA (causal within the q_len queries) + logsumexp on gathered rows."""
    case = inputs.make_case([3, 33, 64, 100], num_heads=4, q_len=3, seed=14)
    o, lse = _run(case, lib_path)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        kfull = _dec(_gather(case, b, L))                      # [L, 576]
        qb = _dec(case.q[b]).permute(1, 0, 2).contiguous()      # [H, q, 576]
        k = kfull.unsqueeze(0).expand(case.num_heads, L, inputs.D_QK).contiguous()
        v = kfull[:, :inputs.D_V].unsqueeze(0).expand(case.num_heads, L, inputs.D_V).contiguous()
        pos = torch.arange(L)
        jj = torch.arange(case.q_len).unsqueeze(1)
        mask = pos.unsqueeze(0) <= (L - case.q_len + jj)        # [q, L]
        out = torch.nn.functional.scaled_dot_product_attention(
            qb, k, v, attn_mask=mask, scale=F32_SCALE)          # [H, q, 512]
        scores = (qb @ k.transpose(1, 2)) * F32_SCALE
        scores = scores.masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(scores, dim=-1)               # [H, q]
        for j in range(case.q_len):
            for h in range(case.num_heads):
                r = (b * case.q_len + j) * case.num_heads + h
                np.testing.assert_allclose(o[r], out[h, j].numpy(), rtol=1e-12, atol=1e-12)
                assert abs(lse[r] - float(ref_lse[h, j])) <= 1e-12 * max(1.0, abs(lse[r]))


def pin_page_permutation(lib_path=None):
    """Moving physical pages (and their block-table entries) changes nothing, bitwise."""
    case = inputs.make_case([70, 129], num_heads=3, q_len=2, seed=15)
    o1, l1 = _run(case, lib_path)
    g = torch.Generator().manual_seed(99)
    P = case.num_pages
    perm = torch.randperm(P, generator=g)           # new position of old page p
    kv2 = torch.empty_like(case.kv)
    kv2[perm] = case.kv
    bt2 = perm.to(torch.int32)[case.block_table.to(torch.int64)]
    case2 = inputs.Case(q=case.q, kv=kv2, block_table=bt2, kv_lens=case.kv_lens,
                        q_len=case.q_len, num_heads=case.num_heads)
    o2, l2 = _run(case2, lib_path)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def pin_causal_prefix(lib_path=None):
    """Query j of a q_len-token step equals a q_len = 1 step over KV[0 .. L - q_len + j]."""
    case = inputs.make_case([96, 45], num_heads=2, q_len=4, seed=16)
    o, lse = _run(case, lib_path)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        for j in range(case.q_len):
            n = L - case.q_len + j + 1
            single = inputs.Case(q=case.q[b:b + 1, j:j + 1].contiguous(), kv=case.kv,
                                 block_table=case.block_table[b:b + 1].contiguous(),
                                 kv_lens=torch.tensor([n], dtype=torch.int32), q_len=1,
                                 num_heads=case.num_heads)
            o1, l1 = _run(single, lib_path)
            for h in range(case.num_heads):
                r = (b * case.q_len + j) * case.num_heads + h
                assert np.array_equal(o[r], o1[h]) and lse[r] == l1[h], (b, j, h)


def pin_split_merge(lib_path=None):
    """Page-aligned key ranges run as separate requests, merged in fp64 with
    weights exp(LSE_s - LSE), reproduce the unsplit row (the split-KV identity)."""
    L = 200
    case = inputs.make_case([L], num_heads=2, q_len=1, seed=17)
    o, lse = _run(case, lib_path)
    for bounds in ([0, 32, 200], [0, 64, 96, 160, 200], [0, 192, 200]):
        outs, lses = [], []
        for a, e in zip(bounds[:-1], bounds[1:]):
            sub = inputs.Case(q=case.q, kv=case.kv,
                              block_table=case.block_table[:, a // 32:].contiguous(),
                              kv_lens=torch.tensor([e - a], dtype=torch.int32), q_len=1,
                              num_heads=case.num_heads)
            os_, ls_ = _run(sub, lib_path)
            outs.append(os_)
            lses.append(ls_)
        lses = np.stack(lses)                       # [S, rows]
        tot = np.logaddexp.reduce(lses, axis=0)
        w = np.exp(lses - tot)                      # [S, rows]
        merged = sum(w[s][:, None] * outs[s] for s in range(len(outs)))
        np.testing.assert_allclose(merged, o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(tot, lse, rtol=1e-13, atol=1e-13)


def pin_bounds_and_dominant(lib_path=None):
    """max s <= LSE <= max s + ln n; one overwhelming key pulls O onto its V row."""
    case = inputs.make_case([300], num_heads=2, q_len=1, seed=18)
    o, lse = _run(case, lib_path)
    kfull = _dec(_gather(case, 0, 300))
    for h in range(2):
        s = (kfull @ _dec(case.q[0, 0, h])) * F32_SCALE
        assert float(s.max()) <= lse[h] <= float(s.max()) + math.log(300) + 1e-12
    # make key 123 dominant for head 0: q = that key's codes, large scale
    case.q[0, 0, 0] = _gather(case, 0, 300)[123]
    o, lse = _run(case, lib_path, softmax_scale=10.0)
    v123 = _dec(_gather(case, 0, 300)[123, :inputs.D_V]).numpy()
    np.testing.assert_allclose(o[0], v123, rtol=0, atol=1e-6)


# ---- attention sinks: one extra logit per head in the softmax denominator --------------

def pin_sinks_equal_scores(lib_path=None):
    """softmax_scale = 0 makes every score 0; with sink sigma the closed forms are
    O = output_scale * sum(V) / (n + e^sigma) and LSE = ln(n + e^sigma)."""
    case = inputs.make_case([40, 7], num_heads=2, q_len=1, seed=21, output_scale=1.25)
    for sig in (-2.0, 0.0, 3.5, 40.0):
        sinks = [sig, sig - 1.0]
        o, lse = _run(case, lib_path, softmax_scale=0.0, sinks=sinks)
        for b in range(case.batch):
            n = int(case.kv_lens[b])
            vsum = _dec(_gather(case, b, n)[:, :inputs.D_V]).sum(dim=0).numpy()
            for h in range(2):
                r = b * 2 + h
                denom = n + math.exp(sinks[h])
                ref_o = 1.25 * vsum / denom
                np.testing.assert_allclose(o[r], ref_o, rtol=1e-13,
                                           atol=1e-13 * np.abs(ref_o).max())
                ref = math.log(denom)
                assert abs(lse[r] - ref) <= 1e-14 * max(1.0, abs(ref)), (sig, h, lse[r], ref)


def pin_sinks_logaddexp(lib_path=None):
    """Against the sink-free oracle: LSE_sink = logaddexp(LSE, sigma_h) and
    O_sink = O * exp(LSE - LSE_sink), per head, up to a sink far above every score
    (sigma = 1000, where exp(sigma) alone overflows fp64); sigma = -inf changes no bit."""
    case = inputs.make_case([150, 33, 64], num_heads=5, q_len=2, seed=22)
    o0, l0 = _run(case, lib_path)
    sinks = np.array([-1.0, 2.0, 5.0, 30.0, 1000.0])
    o1, l1 = _run(case, lib_path, sinks=sinks)
    h = np.arange(o0.shape[0]) % case.num_heads
    ref_l = np.logaddexp(l0, sinks[h])
    np.testing.assert_allclose(l1, ref_l, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o1, o0 * np.exp(l0 - ref_l)[:, None], rtol=1e-11, atol=1e-15)
    o2, l2 = _run(case, lib_path, sinks=np.full(case.num_heads, -np.inf))
    assert np.array_equal(o2, o0) and np.array_equal(l2, l0)


def pin_sinks_mpmath(lib_path=None):
    """Tiny inputs with sinks against 50-digit arithmetic, no max subtraction."""
    import mpmath
    mpmath.mp.dps = 50
    case = inputs.make_case([5, 3], num_heads=2, q_len=1, seed=23)
    sinks = [0.75, -3.0]
    o, lse = _run(case, lib_path, sinks=sinks)
    sc = mpmath.mpf(F32_SCALE)
    for b in range(case.batch):
        n = int(case.kv_lens[b])
        rows = _dec(_gather(case, b, n)).tolist()
        for h in range(2):
            r = b * 2 + h
            qv = _dec(case.q[b, 0, h]).tolist()
            es = [mpmath.exp(sc * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c)
                                               for a, c in zip(qv, rows[i]))) for i in range(n)]
            tot = mpmath.fsum(es) + mpmath.exp(mpmath.mpf(sinks[h]))
            ref_lse = float(mpmath.log(tot))
            assert abs(lse[r] - ref_lse) <= 1e-13 * max(1.0, abs(ref_lse))
            for d in range(0, inputs.D_V, 11):
                ref = float(mpmath.fsum(es[i] * rows[i][d] for i in range(n)) / tot)
                assert abs(o[r, d] - ref) <= 1e-13 * max(1.0, abs(ref)), (d, o[r, d], ref)


# ---- BF16 rounding and the MXFP8 output form ----------------------------------------

def _bf16_grid_values(seed):
    """fp32-exact test values across the BF16 range: random, exact ties (halfway
    between BF16 neighbours), subnormals, and values that overflow."""
    g = np.random.default_rng(seed)
    mant = g.integers(0, 1 << 16, size=4000).astype(np.float64)
    expo = g.integers(-140, 120, size=4000)
    rnd = np.ldexp(1.0 + mant / 65536.0, expo) * np.where(g.random(4000) < 0.5, -1, 1)
    # halfway points: BF16 value + half a step (odd and even neighbours)
    base = np.ldexp(1.0 + np.arange(128) / 128.0, 3)
    ties = np.concatenate([base + 2.0 ** -5, -(base + 2.0 ** -5)])
    sub = np.ldexp(np.arange(1, 64, dtype=np.float64), -140)  # BF16 subnormal range
    big = np.array([3.3895313892515355e38, 3.39e38, -3.4e38])
    return np.concatenate([rnd, ties, sub, big]).astype(np.float32).astype(np.float64)


def pin_bf16_rounding(lib_path=None):
    """The oracle's BF16 rounding against torch's float -> bfloat16 cast (a separate
    library routine) on fp32-exact values, ties and subnormals included."""
    x = _bf16_grid_values(31)
    ours = oracle.round_bf16(x, lib_path)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:5]
    assert oracle.round_bf16([1.0 + 2.0 ** -8], lib_path)[0] == 1.0        # tie -> even
    assert oracle.round_bf16([1.0 + 3 * 2.0 ** -8], lib_path)[0] == 1.0 + 2.0 ** -6


def _mx_blocks(seed):
    """Rows of BF16 values whose 32-element blocks span the interesting cases."""
    g = np.random.default_rng(seed)
    rows = []
    for k in (-140, -130, -20, -3, 0, 5, 9, 40, 119):
        x = g.standard_normal(512) * 2.0 ** k
        rows.append(x)
    x = np.zeros(512)
    x[0:32] = 448.0                                   # amax exactly 448 * 2^0
    x[32:64] = 448.0 * 2.0 ** 5                        # 448 * 2^5
    x[64] = 448.0 * (1 + 2.0 ** -7)                    # next BF16 above 448
    x[96] = 1.75                                      # 448 * 2^-8
    x[128] = 1.875                                    # just above
    x[160:192] = -g.random(32) * 3.0                  # negative block
    x[192:224] = 0.0                                  # all zero
    x[224] = -0.0
    x[256:288] = np.ldexp(1.0 + np.arange(32) / 8.0, -3)
    x[288] = 1.7421875                                # the BF16 value just below 1.75
    x[289] = -0.0                                     # -0 in a block that is not saturated
    rows.append(x)
    y = np.zeros(512)                                 # the low end of the E8M0 range
    y[0:4] = [2.0 ** -125, -2.0 ** -130, 0.0, -0.0]   # scale byte 0: the block saturates
    y[32] = 1.75 * 2.0 ** -119                        # = 448 * 2^-127: scale byte 1
    y[33] = -2.0 ** -133
    y[64] = 1.7421875 * 2.0 ** -119                   # just below: scale byte 0
    y[65] = -0.0
    y[96] = 2.0 ** -133                               # the smallest BF16 subnormal
    rows.append(y)
    return oracle.round_bf16(np.stack(rows))


def pin_mxfp8(lib_path=None):
    """MXFP8 of BF16 rows (PR #17441 "m3 decode perf clean", commit messages on the MXFP8
    quantize tile and on its scale byte 0): every scale is the smallest power of two 2^e
    with amax < 448 * 2^e, strictly, so amax = 1.75 * 2^k takes the next exponent (from
    frexp, a different route), clamped to [-127, 127]; a block of scale byte 0 saturates
    (non-zero elements to +-448, zeros stay zeros); every other element is torch's RNE
    float8_e4m3fn cast of x / 2^e; hand cases pin the edges."""
    x = _mx_blocks(41)
    codes, scales = oracle.mxfp8_quantize(x, lib_path)
    xb = x.reshape(x.shape[0], 16, 32)
    amax = np.abs(xb).max(axis=2)
    # frexp: amax = f * 2^k with f in [0.5, 1); 448 = 0.875 * 2^9, so amax < 448 * 2^e
    # first holds at e = k - 9 when f < 0.875, else at e = k - 8
    f, k = np.frexp(amax)
    e_ref = np.where(f < 0.875, k - 9, k - 8)
    e_ref = np.where(amax == 0, -127, np.clip(e_ref, -127, 127))
    assert np.array_equal(scales.astype(np.int64) - 127, e_ref), "block scales"
    y = xb / np.ldexp(1.0, e_ref)[:, :, None]
    ref = torch.from_numpy(y.reshape(x.shape).astype(np.float32)).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy().reshape(xb.shape)
    sat = np.where(xb != 0, 0x7E, 0x00) | np.where(np.signbit(xb), 0x80, 0x00)
    ref = np.where((e_ref == -127)[:, :, None], sat, ref).astype(np.uint8).reshape(x.shape)
    assert np.array_equal(codes, ref), np.argwhere(codes != ref)[:5]
    hand, low = codes[-2], codes[-1]
    sh, sl = scales[-2], scales[-1]
    assert sh[0] == 128 and (hand[0:32] == 0x76).all()       # 448 -> 2^1, 224 -> code 0x76
    assert sh[1] == 133 and (hand[32:64] == 0x76).all()
    assert sh[2] == 128 and hand[64] == 0x76                 # 452 / 2 = 226 -> 224
    assert sh[3] == 120 and hand[96] == 0x76                 # 1.75 = 448 * 2^-8 -> 2^-7
    assert sh[4] == 120                                      # 1.875 > 1.75
    assert sh[6] == 0 and (hand[192:224] == 0).all()         # zero block: byte 0, zeros
    assert hand[224] == 0x80                                 # -0 keeps its sign
    assert sh[9] == 119 and hand[288] == 0x7E                # 1.7421875 < 1.75: 2^-8, 446 -> 448
    assert hand[289] == 0x80
    assert sl[0] == 0 and list(low[0:4]) == [0x7E, 0xFE, 0x00, 0x80]   # saturated block
    assert sl[1] == 1 and low[32] == 0x76                    # 1.75 * 2^-119 -> 2^-126
    assert sl[2] == 0 and low[64] == 0x7E and low[65] == 0x80
    assert sl[3] == 0 and low[96] == 0x7E                    # smallest subnormal saturates
    # dequantization error: at most half an E4M3 step of x / 2^e (unsaturated blocks)
    live = e_ref > -127
    deq = oracle.e4m3_table(lib_path)[codes].reshape(xb.shape) * np.ldexp(1.0, e_ref)[:, :, None]
    ya = np.abs(y)
    step = np.where(ya >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(ya, 1e-300))).astype(int) - 3),
                    2.0 ** -9)
    ok = np.abs(deq - xb) <= 0.5 * step * np.ldexp(1.0, e_ref)[:, :, None] * (1 + 1e-15)
    assert ok[live].all()


# ---- key windows (kv_bounds) ------------------------------------------------------------

def _rebuilt_request(case, b, k0, k1, j):
    """A one-request, q_len = 1 case holding only the cached tokens k0 .. k1-1 of request
    b (gathered with torch indexing into fresh pages) and query token j of b."""
    tok = torch.arange(k0, k1)
    pages = case.block_table[b].to(torch.int64)[tok // inputs.PAGE]
    rows = case.kv[pages, tok % inputs.PAGE]
    n = k1 - k0
    npg = (n + inputs.PAGE - 1) // inputs.PAGE
    kv = torch.zeros((npg, inputs.PAGE, inputs.D_QK), dtype=case.kv.dtype)
    kv.view(-1, inputs.D_QK)[:n] = rows
    return inputs.Case(q=case.q[b:b + 1, j:j + 1].clone(), kv=kv,
                       block_table=torch.arange(npg, dtype=torch.int32)[None],
                       kv_lens=torch.tensor([n], dtype=torch.int32), q_len=1,
                       num_heads=case.num_heads, output_scale=case.output_scale,
                       kv_dtype=case.kv_dtype)


def _windows_case(kv_dtype="e4m3"):
    case = inputs.make_case([300, 97, 1000, 64], num_heads=3, q_len=4, seed=61,
                            output_scale=0.8, kv_dtype=kv_dtype)
    # page-unaligned starts and ends, a window past the causal frontier, one past L, one
    # whole request, one that only some queries reach, and an empty one
    bounds = torch.tensor([[37, 250], [-5, 500], [512, 998], [70, 70]], dtype=torch.int32)
    return case, bounds


def pin_kv_bounds_rebuilt(lib_path=None):
    """[issue #20510, Repro 1: kv_bounds] A row confined to [start, end) equals, bit for
    bit, the unbounded oracle on a cache rebuilt (by torch indexing) from just the keys it
    may see, start .. min(end, L - q_len + j + 1) - 1. Block-table entries of pages wholly
    outside every window point at a NaN page, which must never be read."""
    for dt in ("e4m3", "bf16"):
        case, bounds = _windows_case(dt)
        bt = case.block_table.clone()
        nan_page = case.kv.shape[0] - 1          # the poison page of make_case
        for b in range(case.batch):
            lo = max(0, int(bounds[b, 0]))
            for p in range(bt.shape[1]):
                if 32 * (p + 1) <= lo:
                    bt[b, p] = nan_page
        poisoned = inputs.Case(q=case.q, kv=case.kv, block_table=bt, kv_lens=case.kv_lens,
                               q_len=case.q_len, num_heads=case.num_heads,
                               output_scale=case.output_scale, kv_dtype=dt)
        o, lse = oracle.mla_decode(poisoned.q, poisoned.kv, bt, case.kv_lens, q_len=case.q_len,
                                   num_heads=case.num_heads, softmax_scale=F32_SCALE,
                                   output_scale=case.output_scale, lib_path=lib_path,
                                   kv_dtype=dt, kv_bounds=bounds)
        assert np.isfinite(o).all(), "a key outside its window was read"
        H, Q = case.num_heads, case.q_len
        for b in range(case.batch):
            L = int(case.kv_lens[b])
            for j in range(Q):
                k0 = max(0, int(bounds[b, 0]))
                k1 = min(int(bounds[b, 1]), L - Q + j + 1)
                rows = [(b * Q + j) * H + h for h in range(H)]
                if k1 <= k0:
                    assert (o[rows] == 0).all() and np.isneginf(lse[rows]).all()
                    continue
                sub = _rebuilt_request(case, b, k0, k1, j)
                o_r, lse_r = _run(sub, lib_path)
                assert np.array_equal(o[rows], o_r), (dt, b, j)
                assert np.array_equal(lse[rows], lse_r), (dt, b, j)


def pin_kv_bounds_whole_and_empty(lib_path=None):
    """A window covering every key gives the unbounded result bit for bit; an empty one
    gives O = 0 and LSE = -inf, or LSE = the sink's logit when the row has a sink."""
    case = inputs.make_case([300, 97], num_heads=2, q_len=3, seed=62)
    o0, l0 = _run(case, lib_path)
    for bounds in ([[0, 300], [0, 97]], [[-7, 10 ** 6], [0, 97]]):
        o, l = oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=3,
                                 num_heads=2, softmax_scale=F32_SCALE, lib_path=lib_path,
                                 kv_bounds=np.array(bounds, np.int32))
        assert np.array_equal(o, o0) and np.array_equal(l, l0)
    sinks = np.array([1.5, -2.0])
    for sk in (None, sinks):
        o, l = oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=3,
                                 num_heads=2, softmax_scale=F32_SCALE, lib_path=lib_path,
                                 sinks=sk, kv_bounds=np.array([[5, 5], [90, 40]], np.int32))
        assert (o == 0).all()
        ref = np.full(12, -np.inf) if sk is None else np.tile(sinks, 6)
        assert np.array_equal(l, ref), l


def pin_kv_bounds_mpmath(lib_path=None):
    """Tiny windows against 50-digit arithmetic (no max subtraction), with the causal
    frontier inside the window for some queries."""
    import mpmath
    mpmath.mp.dps = 50
    case = inputs.make_case([9, 40], num_heads=2, q_len=3, seed=63, output_scale=0.5)
    bounds = np.array([[2, 8], [33, 39]], np.int32)
    o, lse = oracle.mla_decode(case.q, case.kv, case.block_table, case.kv_lens, q_len=3,
                               num_heads=2, softmax_scale=F32_SCALE, output_scale=0.5,
                               lib_path=lib_path, kv_bounds=bounds)
    sc = mpmath.mpf(F32_SCALE)
    for b in range(2):
        L = int(case.kv_lens[b])
        rows_all = _dec(_gather(case, b, L)).tolist()
        for j in range(3):
            keys = [i for i in range(L) if bounds[b, 0] <= i < bounds[b, 1] and i <= L - 3 + j]
            for h in range(2):
                r = (b * 3 + j) * 2 + h
                qv = _dec(case.q[b, j, h]).tolist()
                es = [mpmath.exp(sc * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c)
                                                  for a, c in zip(qv, rows_all[i]))) for i in keys]
                tot = mpmath.fsum(es)
                assert abs(lse[r] - float(mpmath.log(tot))) <= 1e-13 * max(1.0, abs(lse[r]))
                for d in range(0, inputs.D_V, 11):
                    ref = float(mpmath.mpf("0.5") *
                                mpmath.fsum(e * rows_all[i][d] for e, i in zip(es, keys)) / tot)
                    assert abs(o[r, d] - ref) <= 1e-13 * max(1.0, abs(ref)), (b, j, h, d)


# ---- the BF16 cache variant ---------------------------------------------------------

def pin_bf16_table(lib_path=None):
    """All 65536 BF16 bit patterns against torch's bfloat16 -> float64 conversion."""
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([oracle.bf16_decode(c, lib_path) for c in range(65536)])
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    assert (nan_o == nan_r).all() and nan_o.sum() == 2 * 127
    assert np.array_equal(ours[~nan_o], ref[~nan_r])
    assert np.array_equal(np.signbit(ours[~nan_o]), np.signbit(ref[~nan_r]))


def pin_bf16_sdpa(lib_path=None):
    """BF16 cache: fp64 torch SDPA (causal for q > 1) and logsumexp on gathered rows."""
    case = inputs.make_case([3, 40, 97], num_heads=3, q_len=3, seed=51, kv_dtype="bf16",
                            output_scale=0.5)
    o, lse = _run(case, lib_path)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        kfull = _dec_case(case, _gather(case, b, L))
        qb = _dec_case(case, case.q[b]).permute(1, 0, 2).contiguous()
        k = kfull.unsqueeze(0).expand(case.num_heads, L, inputs.D_QK).contiguous()
        v = kfull[:, :inputs.D_V].unsqueeze(0).expand(case.num_heads, L, inputs.D_V).contiguous()
        mask = torch.arange(L).unsqueeze(0) <= (L - case.q_len + torch.arange(case.q_len).unsqueeze(1))
        out = 0.5 * torch.nn.functional.scaled_dot_product_attention(
            qb, k, v, attn_mask=mask, scale=F32_SCALE)
        scores = ((qb @ k.transpose(1, 2)) * F32_SCALE).masked_fill(~mask, float("-inf"))
        ref_lse = torch.logsumexp(scores, dim=-1)
        for j in range(case.q_len):
            for h in range(case.num_heads):
                r = (b * case.q_len + j) * case.num_heads + h
                np.testing.assert_allclose(o[r], out[h, j].numpy(), rtol=1e-12, atol=1e-12)
                assert abs(lse[r] - float(ref_lse[h, j])) <= 1e-12 * max(1.0, abs(lse[r]))


def pin_bf16_closed_forms(lib_path=None):
    """BF16 cache: one key gives O = V_0 exactly and LSE = s_0 (exact rational score,
    to fp64 rounding); q = 0 gives the mean of the visible V rows and LSE = ln n."""
    case = inputs.make_case([1, 1], num_heads=2, q_len=1, seed=52, kv_dtype="bf16")
    o, lse = _run(case, lib_path)
    for b in range(2):
        k = _gather(case, b, 1)[0]
        kv_f = [Fraction(x) for x in _dec_case(case, k).tolist()]
        for h in range(2):
            r = b * 2 + h
            qv = [Fraction(x) for x in _dec_case(case, case.q[b, 0, h]).tolist()]
            s0 = float(Fraction(F32_SCALE) * sum(a * c for a, c in zip(qv, kv_f)))
            assert abs(lse[r] - s0) <= 1e-15 * max(1.0, abs(s0)), (lse[r], s0)
            assert np.array_equal(o[r], _dec_case(case, k[:inputs.D_V]).numpy())
    case = inputs.make_case([37, 64, 5], num_heads=2, q_len=3, seed=53, kv_dtype="bf16")
    case.q.zero_()
    o, lse = _run(case, lib_path)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        for j in range(case.q_len):
            n = L - case.q_len + j + 1
            mean = _dec_case(case, _gather(case, b, n)[:, :inputs.D_V]).mean(dim=0).numpy()
            for h in range(2):
                r = (b * case.q_len + j) * 2 + h
                np.testing.assert_allclose(o[r], mean, rtol=1e-13, atol=1e-13)
                assert abs(lse[r] - math.log(n)) <= 1e-14 * max(1.0, math.log(n))


def pin_bf16_mpmath(lib_path=None):
    """BF16 cache, tiny inputs, against 50-digit arithmetic with no max subtraction."""
    import mpmath
    mpmath.mp.dps = 50
    case = inputs.make_case([4, 9], num_heads=2, q_len=2, seed=54, kv_dtype="bf16")
    o, lse = _run(case, lib_path)
    sc = mpmath.mpf(F32_SCALE)
    for b in range(case.batch):
        L = int(case.kv_lens[b])
        for j in range(case.q_len):
            n = L - case.q_len + j + 1
            rows = _dec_case(case, _gather(case, b, n)).tolist()
            for h in range(2):
                r = (b * case.q_len + j) * 2 + h
                qv = _dec_case(case, case.q[b, j, h]).tolist()
                es = [mpmath.exp(sc * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c)
                                                   for a, c in zip(qv, rows[i])))
                      for i in range(n)]
                tot = mpmath.fsum(es)
                ref_lse = float(mpmath.log(tot))
                assert abs(lse[r] - ref_lse) <= 1e-13 * max(1.0, abs(ref_lse))
                for d in range(0, inputs.D_V, 13):
                    ref = float(mpmath.fsum(es[i] * rows[i][d] for i in range(n)) / tot)
                    assert abs(o[r, d] - ref) <= 1e-13 * max(1.0, abs(ref)), (d, o[r, d], ref)


ALL_PINS = [pin_e4m3_table, pin_single_key, pin_equal_scores, pin_mpmath_bruteforce,
            pin_sdpa, pin_page_permutation, pin_causal_prefix, pin_split_merge,
            pin_bounds_and_dominant, pin_sinks_equal_scores, pin_sinks_logaddexp,
            pin_sinks_mpmath, pin_bf16_rounding, pin_mxfp8, pin_kv_bounds_rebuilt,
            pin_kv_bounds_whole_and_empty, pin_kv_bounds_mpmath, pin_bf16_table, pin_bf16_sdpa,
            pin_bf16_closed_forms, pin_bf16_mpmath]
