// Split-KV partial kernel for MLA decode over a paged FP8 E4M3 cache, gfx950.
//
// What it computes (per request b, split s, block of 16*NT query rows): for every row r
// and the split's key range [t0, t1), the online-softmax state of TensorRT-LLM PR #20380
// "trtllm-gen FMHA: split the KV partials of a row across thread groups in
// fmhaReductionKernel" (Description: per-row max, sum and unnormalised O):
//     m  = an integer >= max_i t_i        (t_i = log2(e) * softmax_scale * q . K_i)
//     l  = sum_i 2^(t_i - m + 8)          (unquantised, for the LSE)
//     l~ = sum_i P~_i,   O = sum_i P~_i V_i
// where P~_i ~ 2^(t_i - m + 8) is the two-term E4M3 form used by the PV matrix product,
// V_i is the 512-byte latent of cached row i, and the causal limit of the MTP verify
// shape applies (issue #20510 "CuTe DSL FP8 MLA decode slower after #19338", Setup).
//
// Design for gfx950: one workgroup per work item (10 wavefronts for one row tile, 16 for
// two), one work item per CU; on plans that would leave CUs idle a work item is a run of
// whole steps of a split, and a fold kernel combines the runs' states.
//  * Page gather, register-staged: loader waves read the split's pages with 16-byte
//    global loads into VGPRs two steps (2 pages each) ahead of use and store them into
//    a 3-stage LDS ring. A page is one contiguous 18 KB block of HBM, so every load
//    instruction reads 1 KB contiguously. In LDS each 576-byte token row is padded to
//    592 bytes, which makes the row-strided operand reads (16 rows at once) hit
//    distinct banks. Block-table entries are read with scalar loads one step early.
//  * QK^T: QK wave (page p, row tile rt) forms the two 16-token tiles of S^T = K Q^T of
//    its page on v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3, fp32 accumulate), K from LDS
//    and Q^T resident in VGPRs; the 576-wide dot is 4 full MFMAs plus one whose rope
//    half is zero in both operands. Row tiles of a work item share every staged page,
//    so KV is read from HBM once per 32 query rows.
//  * Softmax (exp2 domain, in the QK wave): per (row, page) c = ceil(max t over the
//    page), x = 2^(t - c + 8) in (0, 256], P~ = hi + lo/16 with hi = e4m3(x),
//    lo = e4m3(16 (x - hi)). P~ depends only on the page's own scores, so a token gets
//    bit-identical P~ under every split plan (splits hold whole pages), and the QK
//    waves never need the running maximum.
//  * PV (PV waves): the row max is kept on integers, m = max over pages of c, and the
//    factor 2^(c - m) rides in the MFMA's E8M0 block scale; every rescale is an exact
//    power of two. One scaled MFMA covers 64 tokens of both terms: A bytes 0-15 hold hi,
//    bytes 16-31 lo of the same 16 tokens; K-block b = (term b >> 1, page b & 1) takes
//    its scale from lane row + 16 b, i.e. 2^(c_page - m) for hi and 2^(c_page - m - 4)
//    for lo. V is the same LDS rows as K (never a second HBM read), gathered transposed
//    with ds_read_b64_tr_b8. l~ comes from one extra MFMA against a tile of ones.
//  * Skewed single-barrier pipeline: iteration s does QK/softmax of step s + 1 and PV of
//    step s concurrently (P~ and the page maxima are double-buffered), while loaders
//    store step s + 2 and load step s + 4.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kStepPages = 2;
constexpr int kRowLds = kDQK + 16;                    // 592: padded token row in LDS
constexpr int kPageLds = kPage * kRowLds;             // 18944
constexpr int kStepLds = kStepPages * kPageLds;       // 37888
constexpr int kStages = 3;
constexpr int kChunksPerStep = kStepPages * kPageBytes / 1024;  // 36 wave-wide 16 B loads
constexpr int kPRow = 144;                            // P~ row: 64 hi, 64 lo, 16 pad
constexpr int kOnesE4M3 = 0x38383838;                 // four E4M3 1.0

// Wave roles. Every wave is one of: QK (one page of the step for one row tile: wave
// w < 2 NT takes page w & 1 and row tile w >> 1), loader (36 / kLdWaves chunks of 1 KB
// per step), PV (8 of the 32 16-dim tiles of O for one row tile; four PV waves per row
// tile, so a PV wave holds the same state whatever NT is).
//  NT = 1: 10 waves (2-3 per SIMD, 168 VGPRs): 2 QK, 4 loaders, 4 PV. Four loaders of
//          9 KB per step keep the gather as busy as six of 6 KB and leave the SIMDs
//          fewer waves (measured 1-4% faster than six).
//  NT = 2: 16 waves (4 per SIMD, 128 VGPRs): 4 QK, 4 loaders, 8 PV.
template <int NT>
struct Roles {
  static_assert(NT == 1 || NT == 2, "row tiles per workgroup");
  static constexpr int kWaves = NT == 1 ? 10 : 16;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kQK = 2 * NT;
  static constexpr int kLdFirst = 2 * NT;
  static constexpr int kLdWaves = 4;
  static constexpr int kPVFirst = kLdFirst + kLdWaves;
  static constexpr int kDimTiles = 32 * NT / (kWaves - kPVFirst);  // 8: dim tiles per PV wave
  static constexpr int kDimSlices = 32 / kDimTiles;                // 4 PV waves per row tile
  static_assert(kDimSlices * NT == kWaves - kPVFirst, "PV waves cover every (row tile, dim slice)");
  static constexpr int kMaxLd = kChunksPerStep / kLdWaves;    // 9
  // Waves w, w + 4, w + 8 share a SIMD (a workgroup's waves are dealt round-robin).
  // NT = 2: QK 0-3, loaders 4-7, PV 8-15, the same mix on every SIMD. NT = 1: QK 0-1,
  // PV 2-3 and 6-7, loaders 4-5 and 8-9, so that the two SIMDs that run a QK wave get
  // two loaders beside it (the lightest role) and the other two a pair of PV waves;
  // QK, loaders and PV 0-5 in that order left the QK SIMDs with a loader and a PV wave
  // each and the others with a loader and a PV wave half idle.
  enum { kRoleQK, kRoleLd, kRolePV };
  static __device__ __forceinline__ int role(int w) {
    if (w < kQK) return kRoleQK;
    if (NT == 2) return w < kPVFirst ? kRoleLd : kRolePV;
    return (w & 3) >= 2 && w < 8 ? kRolePV : kRoleLd;
  }
  // index among the loaders (0 .. kLdWaves - 1) and among the PV waves
  static __device__ __forceinline__ int ld_index(int w) {
    return NT == 2 ? w - kLdFirst : (w < 8 ? w - 4 : w - 6);
  }
  static __device__ __forceinline__ int pv_index(int w) {
    return NT == 2 ? w - kPVFirst : (w < 6 ? w - 2 : w - 4);
  }
};

template <int NT>
struct __attribute__((aligned(16))) Smem {
  uint8_t pages[kStages][kStepLds];
  uint8_t ptile[2][NT * kTileRows * kPRow];
  float2 cl[2][NT * kTileRows][kStepPages];  // per (row, page): (c, sum of x)
};

__device__ __forceinline__ float ldexp_int(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }

__device__ __forceinline__ v4i ld16(const uint8_t* base, int off) {
  return *(const v4i*)(base + off);
}

__device__ __forceinline__ v8i cat8(v4i a, v4i b) {
  return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

// Workgroup barrier ordering LDS traffic (the global loads in flight are not waited on).
__device__ __forceinline__ void block_sync_lds() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 2^(a - b) for integer-valued a <= b; 0 when a is -inf.
__device__ __forceinline__ float pow2_diff(float a, float b) {
  return a == -INFINITY ? 0.f : ldexp_int(1.f, (int)(a - b));
}

// What every wave of a work item knows.
struct Item {
  const PlanDev* P;
  const uint8_t* q;
  const uint8_t* kv;
  const int32_t* btb;
  float* ws_o;
  float* ws_stats;
  float scale_log2;
  int b, part, L, t0, t1, row0, p_first, p_end, nsteps;  // keys [t0, t1), pages [p_first, p_end)
  int qb;  // query tokens of the request (ragged batches), <= q_len
  int lane, w, g, l16;
};

constexpr int kNoKey = -0x40000000;  // causal limit of a row that sees no key

// One wave's whole life: prologue, then 1 + nsteps barriers like every other wave.
// kNB: steps of page data each loader holds in registers (loads in flight per loader):
// 2 when the grid fills the chip, 3 for grids of fewer work items than CUs, where each
// CU must pull more bytes per second and only the latency of HBM limits it.
template <int NT, int kNB, bool kDoQK, bool kDoLd, bool kDoPV>
__device__ __forceinline__ void wave_main(const Item& it, Smem<NT>& sm) {
  static_assert(kNB == 2 || kNB == 3, "loader buffers (the tail below runs < 3 steps)");
  using R = Roles<NT>;
  const PlanDev& P = *it.P;
  const int lane = it.lane, w = it.w, g = it.g, l16 = it.l16;
  const int nsteps = it.nsteps, p_first = it.p_first, p_end = it.p_end, t1 = it.t1, L = it.L;
  const int t0 = it.t0;  // a key window can start inside the first page
  const int row0 = it.row0;

  // ---------------- QK role: QK^T + softmax of (page w & 1, row tile w >> 1) ----------------
  const int qk_rt = w >> 1, qk_page = w & 1;
  v8i qf[kDoQK ? 5 : 1];
  int k_base[2] = {0, 0};
  int lim_q = 0, lim_all = 0, rope_off = 0;
  if (kDoQK) {
    // Q^T fragments: lane (row l16, group g) holds bytes [32g, 32g + 32) of each 128-byte
    // K-step of its row; the rope step uses groups 0-1 only.
    const int qrow = row0 + qk_rt * kTileRows + l16;
    const bool qrow_valid = qrow < P.rows;
    const uint8_t* qp = it.q + ((int64_t)it.b * P.rows + (qrow_valid ? qrow : 0)) * kDQK;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      v4i a = ld16(qp, 128 * c4 + 32 * g);
      v4i c = ld16(qp, 128 * c4 + 32 * g + 16);
      if (!qrow_valid) { a = 0; c = 0; }
      qf[c4] = cat8(a, c);
    }
    const int gg = g & 1;
    v4i a = ld16(qp, 512 + 32 * gg);
    v4i c = ld16(qp, 512 + 32 * gg + 16);
    if (!qrow_valid || g >= 2) { a = 0; c = 0; }
    qf[kDoQK ? 4 : 0] = cat8(a, c);
    // causal limit of the row: query j sees tokens < L - q_len + j + 1
    // causal limit of the row: query j of a request with qb queries sees tokens
    // < L - qb + j + 1; rows past the request's queries see none
    const int qb = it.qb;
    const int jq = qrow_valid ? qrow / P.heads : 0;
    lim_q = jq < qb ? min(t1, L - qb + jq + 1) : kNoKey;
    // below this token no row of the work item needs a mask
    const int j_first = min(row0, P.rows - 1) / P.heads;
    const int j_last = (min(row0 + NT * kTileRows, P.rows) - 1) / P.heads;
    lim_all = j_last >= qb ? kNoKey : min(t1, L - qb + j_first + 1);
    // K operand: token row n = 16 tt + l16 of the page, bytes 128 c4 + 32 g (+16)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      k_base[tt] = qk_page * kPageLds + (16 * tt + l16) * kRowLds + 32 * g;
    rope_off = 512 + 32 * (g & 1) - 32 * g;
  }

  auto qk_step = [&](int st) {
    const uint8_t* stage = sm.pages[st % kStages];
    v4f sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      v4f a4 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const v8i kf = cat8(ld16(stage, k_base[tt] + 128 * c4), ld16(stage, k_base[tt] + 128 * c4 + 16));
        a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[kDoQK ? c4 : 0], a4, 0, 0, 0, 127, 0, 127);
      }
      v4i ra = ld16(stage, k_base[tt] + rope_off);
      v4i rb = ld16(stage, k_base[tt] + rope_off + 16);
      if (g >= 2) { ra = 0; rb = 0; }
      sacc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat8(ra, rb), qf[kDoQK ? 4 : 0], a4, 0, 0, 0, 127, 0, 127);
    }
    // lane holds S[row l16][token 16 tt + 4g + jj] of the page
    const int tok_page = (p_first + st * kStepPages + qk_page) * kPage;
    const bool need_mask = tok_page + kPage > lim_all || tok_page < t0;
    float t[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float v = sacc[tt][jj] * it.scale_log2;
        const int tok = tok_page + 16 * tt + 4 * g + jj;
        if (need_mask && (tok >= lim_q || tok < t0)) v = -INFINITY;
        t[tt][jj] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float c = ceilf(mx);  // -inf when no key of the page is visible to the row
    const float off = 8.f - (c == -INFINITY ? 0.f : c);
    float x[2][4];
    float xs = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        x[tt][jj] = exp2f(t[tt][jj] + off);  // exp2(-inf) = 0
        xs += x[tt][jj];
      }
    xs += __shfl_xor(xs, 16);
    xs += __shfl_xor(xs, 32);
    uint8_t* prow = sm.ptile[st & 1] + (qk_rt * kTileRows + l16) * kPRow + qk_page * kPage + 4 * g;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[tt][0], x[tt][1], 0, false);
      hw = __builtin_amdgcn_cvt_pk_fp8_f32(x[tt][2], x[tt][3], hw, true);
      const float h0 = __builtin_amdgcn_cvt_f32_fp8(hw, 0);
      const float h1 = __builtin_amdgcn_cvt_f32_fp8(hw, 1);
      const float h2 = __builtin_amdgcn_cvt_f32_fp8(hw, 2);
      const float h3 = __builtin_amdgcn_cvt_f32_fp8(hw, 3);
      int lw = __builtin_amdgcn_cvt_pk_fp8_f32((x[tt][0] - h0) * 16.f, (x[tt][1] - h1) * 16.f, 0, false);
      lw = __builtin_amdgcn_cvt_pk_fp8_f32((x[tt][2] - h2) * 16.f, (x[tt][3] - h3) * 16.f, lw, true);
      *(int*)(prow + 16 * tt) = hw;
      *(int*)(prow + 64 + 16 * tt) = lw;
    }
    if (g == 0) sm.cl[st & 1][qk_rt * kTileRows + l16][qk_page] = make_float2(c, xs);
  };

  // ---------------- loader role ----------------
  static_assert(kChunksPerStep % R::kLdWaves == 0, "every loader issues the same loads");
  const int li = R::ld_index(w);
  constexpr int kLd = kDoLd ? R::kMaxLd : 1;
  // Loader li owns the kLd consecutive 1 KB chunks k = li kLd .. li kLd + kLd - 1 of a
  // step (chunk k = byte 1024 (k % 18) of page k / 18), all within one page, so each
  // load is a scalar page base plus a per-lane offset; lane i moves 16 bytes into padded
  // LDS row n, column c.
  static_assert(18 % (kDoLd ? R::kMaxLd : 1) == 0, "a loader's chunks stay in one page");
  const int ld_page = kDoLd ? (max(li, 0) * kLd) / 18 : 0;
  // byte of page ld_page that lane moves for chunk i: ld_byte0 + 1024 i
  const uint32_t ld_byte0 = (uint32_t)(((max(li, 0) * kLd) % 18) * 1024 + 16 * lane);
  // Page ids of step st; steps past the split's end repeat its last page (those loads
  // keep the loader's loop free of conditions and their data is never read).
  auto page_ids = [&](int st, int64_t* ida, int64_t* idb) {
    const int pa = min(p_first + st * kStepPages, p_end - 1);
    const int pb = min(pa + 1, p_end - 1);
    *ida = it.btb[pa];
    *idb = it.btb[pb];
  };
  auto gload = [&](int64_t ida, int64_t idb, v4i (&buf)[kLd]) {
    const uint8_t* gp = it.kv + (ld_page ? idb : ida) * kPageBytes + ld_byte0;
#pragma unroll
    for (int i = 0; i < kLd; ++i) buf[i] = __builtin_nontemporal_load((const v4i*)(gp + 1024 * i));
  };
  auto lstore = [&](int st, const v4i (&buf)[kLd]) {
    uint8_t* stage = sm.pages[st % kStages] + ld_page * kPageLds;
    uint32_t b0 = ld_byte0;
    __asm__ volatile("" : "+v"(b0));  // recomputed per step: keeps the offsets out of registers
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const uint32_t byte = b0 + 1024 * i;
      const uint32_t n = byte / kDQK;  // row of the page (576-byte rows, 592-byte LDS rows)
      *(v4i*)(stage + byte + (kRowLds - kDQK) * n) = buf[i];
    }
  };

  // ---------------- PV role ----------------
  const int pv_w = R::pv_index(w);
  const int pv_rt = pv_w / R::kDimSlices;  // row tile of the wave
  const int pv_ds = pv_w % R::kDimSlices;  // dims [16 kDimTiles pv_ds, ...)
  // the waves that keep l (dim slice 0) and l~ (dim slice 1) of their row tile: two
  // waves on different SIMDs share the extra work
  const bool pv_own = pv_ds == 0;
  const bool pv_own_t = pv_ds == 1;
  constexpr int kDT = kDoPV ? R::kDimTiles : 1;
  constexpr int kNTp = 1;                  // row tiles per PV wave (rt below is 0)
  v4f acc[kNTp][kDT];
  v4f acc1 = v4f{0.f, 0.f, 0.f, 0.f};  // l~ of row tile pv_rt (pv_own_t): ones product
  float m_c[kNTp][4];  // running max of result rows
  float m_a[kNTp];     // running max of operand rows (row l16 of the tile)
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // l of rows 4g + jj of row tile pv_rt (pv_own)
#pragma unroll
  for (int rt = 0; rt < kNTp; ++rt) {
    m_a[rt] = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) m_c[rt][jj] = -INFINITY;
#pragma unroll
    for (int d = 0; d < kDT; ++d) acc[rt][d] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // transposed V reads: lane (16G + u) names token 16G + 8r + u/2 and the 8-byte half
  // u%2 of a 16-dim chunk; it receives dim 16D + l16 for 8 tokens.
  int tr_base[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int tokstep = 16 * g + 8 * r + (l16 >> 1);
    const int pg = tokstep >> 5, n = tokstep & 31;
    tr_base[r] = pg * kPageLds + n * kRowLds + 8 * (l16 & 1) + 16 * R::kDimTiles * pv_ds;
  }

  auto pv_step = [&](int st) {
    const uint8_t* stage = sm.pages[st % kStages];
    const int pb = st & 1;
    int sa[kNTp];
    v8i pa[kNTp];
#pragma unroll
    for (int rt = 0; rt < kNTp; ++rt) {
      bool rescale = false;
      float alpha[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float2 p0 = sm.cl[pb][(pv_rt + rt) * kTileRows + 4 * g + jj][0];
        const float2 p1 = sm.cl[pb][(pv_rt + rt) * kTileRows + 4 * g + jj][1];
        const float mn = fmaxf(m_c[rt][jj], fmaxf(p0.x, p1.x));
        alpha[jj] = mn == m_c[rt][jj] ? 1.f : pow2_diff(m_c[rt][jj], mn);
        rescale |= mn != m_c[rt][jj];
        if (pv_own)
          lsum[jj] = lsum[jj] * alpha[jj] + p0.y * pow2_diff(p0.x, mn) + p1.y * pow2_diff(p1.x, mn);
        m_c[rt][jj] = mn;
      }
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
        for (int d = 0; d < kDT; ++d) {
          acc[rt][d][0] *= alpha[0]; acc[rt][d][1] *= alpha[1];
          acc[rt][d][2] *= alpha[2]; acc[rt][d][3] *= alpha[3];
        }
        if (pv_own_t) {
          acc1[0] *= alpha[0]; acc1[1] *= alpha[1]; acc1[2] *= alpha[2]; acc1[3] *= alpha[3];
        }
      }
      const float2 a0 = sm.cl[pb][(pv_rt + rt) * kTileRows + l16][0];
      const float2 a1 = sm.cl[pb][(pv_rt + rt) * kTileRows + l16][1];
      m_a[rt] = fmaxf(m_a[rt], fmaxf(a0.x, a1.x));
      const float cp = (g & 1) ? a1.x : a0.x;
      sa[rt] = cp == -INFINITY ? 127 : max(0, 127 + (int)(cp - m_a[rt]) - 4 * (g >> 1));
      const uint8_t* prow = sm.ptile[pb] + ((pv_rt + rt) * kTileRows + l16) * kPRow + 16 * g;
      pa[rt] = cat8(ld16(prow, 0), ld16(prow, 64));
      if (pv_own_t) {
        const v8i ones = v8i{kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3,
                             kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3};
        acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa[rt], ones, acc1, 0, 0, 0, sa[rt], 0, 127);
      }
    }
    // bytes of tokens past the split's end, or before a window's start in the first
    // page, may be poison: zero them (P~ is 0 there)
    uint32_t mk[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    const bool last = st == nsteps - 1;
    if (last) {
      const int valid = t1 - (p_first + st * kStepPages) * kPage;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // byte j of word q4 is token 16 g + 4 q4 + j: the first nb bytes are valid
        const int nb = min(max(valid - (16 * g + 4 * q4), 0), 4);
        mk[q4] = nb >= 4 ? 0xFFFFFFFFu : (1u << (8 * nb)) - 1u;
      }
    }
    if (st == 0 && t0 > p_first * kPage) {
      const int skip = t0 - p_first * kPage;  // tokens of the step before the window
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // the first nb bytes of word q4 are before the window
        const int nb = min(max(skip - (16 * g + 4 * q4), 0), 4);
        mk[q4] &= nb >= 4 ? 0u : ~((1u << (8 * nb)) - 1u);
      }
    }
#pragma unroll
    for (int d = 0; d < kDT; ++d) {
      const v2i b0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(stage + tr_base[0] + 16 * d));
      const v2i b1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(stage + tr_base[1] + 16 * d));
      const int x0 = b0.x & mk[0], x1 = b0.y & mk[1], x2 = b1.x & mk[2], x3 = b1.y & mk[3];
      const v8i vb = v8i{x0, x1, x2, x3, x0, x1, x2, x3};
#pragma unroll
      for (int rt = 0; rt < kNTp; ++rt)
        acc[rt][d] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa[rt], vb, acc[rt][d], 0, 0, 0, sa[rt], 0, 127);
    }
  };

  // ---------------- pipeline ----------------
  // The data of step t is loaded into loader buffer t % kNB at iteration t - 2 - kNB
  // (steps 0 .. kNB + 1 before the loop) and stored to LDS at iteration t - 2, which
  // then loads step t + kNB into the same buffer. QK of step t runs in iteration t - 1
  // (step 0 before the loop), PV of step t in iteration t. The loop body covers kNB
  // steps, so buffer indices are constants; each store waits for its own buffer, the
  // oldest in flight, while the other kNB - 1 stay in flight. The loads are
  // unconditional (steps past the split's end repeat its last page, never read). The
  // last nsteps % kNB (< 3) steps store nothing: their stages were stored by then.
  v4i buf[kNB][kLd];
  int64_t nid_a = 0, nid_b = 0;
  if (kDoLd && nsteps > 0) {
    int64_t ia, ib;
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      page_ids(j, &ia, &ib);
      gload(ia, ib, buf[j]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lstore(j, buf[j]);
      page_ids(kNB + j, &ia, &ib);
      gload(ia, ib, buf[j]);
    }
    page_ids(kNB + 2, &nid_a, &nid_b);
  }
  block_sync_lds();  // steps 0 and 1 stored
  if (kDoQK && nsteps > 0) qk_step(0);
  const int ngroups = nsteps / kNB;
  for (int i = 0; i < ngroups; ++i) {
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const int st = kNB * i + j;
      block_sync_lds();  // stage st + 1 stored, P~(st) ready, PV(st - 1) done everywhere
      if (kDoLd) {
        lstore(st + 2, buf[(j + 2) % kNB]);
        gload(nid_a, nid_b, buf[(j + 2) % kNB]);
        page_ids(st + 3 + kNB, &nid_a, &nid_b);
      }
      // st + 1 < nsteps holds inside a group but for its last step
      if (kDoQK && (j + 1 < kNB || st + 1 < nsteps)) qk_step(st + 1);
      if (kDoPV) pv_step(st);
    }
  }
  for (int st = kNB * ngroups; st < nsteps; ++st) {
    block_sync_lds();
    if (kDoQK && st + 1 < nsteps) qk_step(st + 1);
    if (kDoPV) pv_step(st);
  }

  // ---------------- write the partials ----------------
  if (kDoPV) {
    const int64_t part_row0 = (int64_t)it.part * P.rows;
#pragma unroll
    for (int rt = 0; rt < kNTp; ++rt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = row0 + (pv_rt + rt) * kTileRows + 4 * g + jj;
        if (row < P.rows) {
          float* orow = it.ws_o + (part_row0 + row) * kDV + 16 * R::kDimTiles * pv_ds + l16;
#pragma unroll
          for (int d = 0; d < kDT; ++d) orow[16 * d] = acc[rt][d][jj];
          if (pv_own && l16 == 0)
            *(float2*)(it.ws_stats + (part_row0 + row) * kStatStride) =
                make_float2(m_c[rt][jj], lsum[jj]);
          if (pv_own_t && l16 == 0)
            *(float2*)(it.ws_stats + (part_row0 + row) * kStatStride + 2) =
                make_float2(acc1[jj], 0.f);
        }
      }
    }
  }
}

// kDev: the plan and the softmax scale come from device memory (graph path).
template <int NT, int kNB, bool kDev>
__global__ void __launch_bounds__(Roles<NT>::kThreads, 1)
partial_kernel(const PlanDev Parg, const PlanDev* __restrict__ pdev,
               const float* __restrict__ scale_dev, const uint8_t* __restrict__ q,
               const uint8_t* __restrict__ kv, const int32_t* __restrict__ bt, int64_t bt_stride,
               const int32_t* __restrict__ kv_lens, const int32_t* __restrict__ q_lens,
               const int32_t* __restrict__ kv_bounds, float scale_log2_arg,
               float* __restrict__ ws_o, float* __restrict__ ws_stats) {
  __shared__ Smem<NT> sm;
  const PlanDev& P = kDev ? *pdev : Parg;
  const float scale_log2 = kDev ? *scale_dev * 1.4426950408889634f : scale_log2_arg;
  Item it;
  it.lane = threadIdx.x & 63;
  it.w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
  it.g = it.lane >> 4;
  it.l16 = it.lane & 15;
  int ps, sub, blk;
  if (!work_item(P, blockIdx.x, &ps, &sub, &blk)) return;
  int e = 0;
  {
    int lo = 0, hi = P.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)(P.sorted[mid] >> 8) > ps) hi = mid; else lo = mid + 1;
    }
    e = lo;
  }
  const int b = (int)(P.sorted[e] & 0xFF);
  const int s = ps - (e > 0 ? (int)(P.sorted[e - 1] >> 8) : 0);
  it.P = &P;
  it.q = q;
  it.kv = kv;
  it.btb = bt + (int64_t)b * bt_stride;
  it.ws_o = ws_o;
  it.ws_stats = ws_stats;
  it.scale_log2 = scale_log2;
  it.b = b;
  it.part = ((int)P.part_base[b] + s) * P.subs + sub;  // subs > 1: the sub-range slot
  it.L = min(kv_lens[b], (int)P.kv_len[b]);
  it.qb = q_lens != nullptr ? min(max(q_lens[b], 0), P.q_len) : P.q_len;
  split_keys(P, b, s, it.L, kv_bounds, &it.t0, &it.t1);
  sub_keys(P, sub, &it.t0, &it.t1);
  it.row0 = blk * NT * kTileRows;
  it.p_first = it.t0 / kPage;
  it.p_end = (it.t1 + kPage - 1) / kPage;
  it.nsteps = it.t1 > it.t0 ? (it.p_end - it.p_first + kStepPages - 1) / kStepPages : 0;

  const int w = it.w;
  using R = Roles<NT>;
  const int role = R::role(w);
  if (role == R::kRoleQK) wave_main<NT, kNB, true, false, false>(it, sm);
  else if (role == R::kRoleLd) wave_main<NT, kNB, false, true, false>(it, sm);
  else wave_main<NT, kNB, false, false, true>(it, sm);
}

}  // namespace

namespace {

int launch_partial_kernel(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                          const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                          float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                          const DeviceArgs* dev, const int32_t* q_lens,
                          const int32_t* kv_bounds) {
  const PlanDev& P = plan.dev;
  if (plan.kv_dtype == MLA_KV_BF16 && P.nt > kMaxTilesPerBlock)
    return launch_partial_bf16_wide(plan, q, kv, bt, bt_stride, kv_lens, softmax_scale, ws_o,
                                    ws_stats, stream, dev, q_lens, kv_bounds);
  if (plan.kv_dtype == MLA_KV_BF16)
    return launch_partial_bf16(plan, q, kv, bt, bt_stride, kv_lens, softmax_scale, ws_o, ws_stats,
                               stream, dev, q_lens, kv_bounds);
  if (P.nt > kMaxTilesPerBlock)
    return launch_partial_wide(plan, q, kv, bt, bt_stride, kv_lens, softmax_scale, ws_o, ws_stats,
                               stream, dev, q_lens, kv_bounds);
  const int slots = (P.total_parts * P.subs + 7) / 8;  // graph plans: the capacity
  const dim3 grid(8 * slots * P.tiles);
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const PlanDev* pd = dev ? dev->plan : nullptr;
  const float* sd = dev ? dev->softmax_scale : nullptr;
  hipStream_t st = (hipStream_t)stream;
#define MLA_NARROW_LAUNCH(NT, NB, DEV)                                                       \
  hipLaunchKernelGGL((partial_kernel<NT, NB, DEV>), grid, dim3(Roles<NT>::kThreads), 0, st, P, \
                     pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2,    \
                     ws_o, ws_stats)
  // one row tile and fewer work items than CUs: three steps of loads in flight per
  // loader (the two-tile kernel has no registers to spare for a third buffer)
  if (P.nt == 1 && narrow_underfilled(plan)) {
    if (dev) MLA_NARROW_LAUNCH(1, 3, true); else MLA_NARROW_LAUNCH(1, 3, false);
  } else if (P.nt == 1) {
    if (dev) MLA_NARROW_LAUNCH(1, 2, true); else MLA_NARROW_LAUNCH(1, 2, false);
  } else {
    if (dev) MLA_NARROW_LAUNCH(2, 2, true); else MLA_NARROW_LAUNCH(2, 2, false);
  }
#undef MLA_NARROW_LAUNCH
  return (int)hipGetLastError();
}

}  // namespace

// With dev.subs > 1 the kernels write one partial state per (split, sub-range) into the
// region after the stats, and the fold kernel turns them into the split partials.
int launch_partial(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                   const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                   float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                   const DeviceArgs* dev, const int32_t* q_lens, const int32_t* kv_bounds) {
  if (plan.dev.subs <= 1)
    return launch_partial_kernel(plan, q, kv, bt, bt_stride, kv_lens, softmax_scale, ws_o,
                                 ws_stats, stream, dev, q_lens, kv_bounds);
  float* sub_o = (float*)((uint8_t*)ws_stats + plan.ws_stats_bytes);
  float* sub_stats = (float*)((uint8_t*)sub_o + plan.ws_sub_o_bytes);
  const int rc = launch_partial_kernel(plan, q, kv, bt, bt_stride, kv_lens, softmax_scale,
                                       sub_o, sub_stats, stream, dev, q_lens, kv_bounds);
  if (rc != 0) return rc;
  return launch_fold(plan, sub_o, sub_stats, ws_o, ws_stats, stream, dev);
}

}  // namespace mla
