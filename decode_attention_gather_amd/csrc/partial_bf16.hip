// Split-KV partial kernel for MLA decode over a paged BF16 cache, gfx950.
//
// The BF16 variant that TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower after
// #19338" measures beside the FP8 kernel (Repro 2): q and the cache hold BF16 values,
// a token row is 576 of them (1152 bytes: latent 512 + rope 64), pages hold 32 rows.
// Per (request b, split s, block of 16 NT query rows) it writes the same partial state
// as the FP8 kernels (PR #20380 "trtllm-gen FMHA: split the KV partials of a row across
// thread groups in fmhaReductionKernel", Description: per-row max, sum and unnormalised
// O), so the merge is shared:
//     m  = an integer >= max_i t_i        (t_i = log2(e) * softmax_scale * q . K_i)
//     l  = sum_i 2^(t_i - m + 8)          (unquantised, for the LSE)
//     l~ = sum_i P~_i,   O = sum_i P~_i V_i
// with P~_i the BF16 rounding of 2^(t_i - c + 8), c = ceil of the max over the 16-token
// tile holding token i, times the exact power of two 2^(c - m). P~ of a token depends
// only on its own tile's scores, so every split plan (splits hold whole pages) gives it
// the same bits.
//
// Design for gfx950 (one workgroup per work item, one work item per CU):
//  * Gather: one page (36,864 contiguous bytes of HBM) per pipeline step; loader waves
//    move it with 36 wave-wide 16-byte loads (1 KB each) into VGPRs two steps ahead and
//    store it into a 3-stage LDS ring with each 1152-byte token row padded to 1168 bytes,
//    which spreads the 16 rows of an operand read over distinct LDS banks.
//  * QK^T: QK wave (row tile rt, token tile tt) forms S^T = K Q^T for 16 tokens on 18
//    v_mfma_f32_16x16x32_bf16 (fp32 accumulate, two accumulator chains), K from LDS and
//    Q^T resident in VGPRs.
//  * Softmax (QK wave): per (row, 16-token tile) c = ceil(max t), x = 2^(t - c + 8),
//    P~ = bf16(x) (round to nearest even) to LDS, with (c, sum x, sum P~).
//  * PV (PV waves): running max m on integers; P~ rows from LDS are scaled by 2^(c - m)
//    (exact) before v_mfma_f32_16x16x32_bf16; V is the same LDS rows as K, gathered
//    transposed with ds_read_b64_tr_b16. K position 8 G + 4 tt + j of an MFMA (G = lane
//    group) holds token 16 tt + 4 G + j, which is where the QK wave's result lanes
//    already are and where one transposed read delivers four tokens.
//  * Skewed single-barrier pipeline: iteration s runs QK/softmax of step s + 1 and PV of
//    step s; loaders store step s + 2 and load step s + 4.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kRowB = 2 * kDQK;                     // 1152 bytes per token row
constexpr int kRowLdsB = kRowB + 16;                // 1168: padded row in LDS
constexpr int kPageB = kPage * kRowB;               // 36864 bytes per page
constexpr int kPageLdsB = kPage * kRowLdsB;         // 37376
constexpr int kStages = 3;
constexpr int kChunks = kPageB / 1024;              // 36 wave-wide 16-byte loads per step
constexpr int kKSteps = kDQK / 32;                  // 18 MFMAs of K = 32 per 576-wide dot
constexpr int kPRowB = 80;                          // P~ row: 32 BF16 + 16 bytes of pad
static_assert(kChunks * 1024 == kPageB && kRowB % 16 == 0, "1 KB loads tile a page");

// Wave roles: QK (row tile w >> 1, token tile w & 1), loader (kChunks / kLdWaves
// chunks per step), PV (kDimTiles of the 32 16-dim tiles of O for all NT row tiles).
//  NT = 1: 10 waves: 2 QK, 4 loaders, 4 PV x 8 dim tiles (four loaders of 9 KB keep the
//          gather as busy as six of 6 KB with fewer waves: 8% faster at 96 workgroups).
//  NT = 2: 16 waves: 4 QK, 4 loaders, 8 PV x 4 dim tiles.
template <int NT>
struct BRoles {
  static_assert(NT == 1 || NT == 2, "row tiles per workgroup");
  static constexpr int kWaves = NT == 1 ? 10 : 16;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kQK = 2 * NT;
  static constexpr int kLdFirst = 2 * NT;
  static constexpr int kLdWaves = 4;
  static constexpr int kPVFirst = kLdFirst + kLdWaves;
  static constexpr int kDimTiles = 32 / (kWaves - kPVFirst);  // 8 or 4
  static constexpr int kMaxLd = kChunks / kLdWaves;          // 9
  static_assert(kMaxLd * kLdWaves == kChunks, "every loader issues the same loads");
  // Waves w, w + 4, w + 8 share a SIMD. In order (QK, loaders, PV), one tile puts a
  // QK, a loader and a PV wave on SIMDs 0-1 and a loader and a PV wave on 2-3. kSpread
  // (one tile, grids of fewer work items than CUs): QK 0-1, PV 2-3 and 6-7, loaders 4-5
  // and 8-9, so the QK SIMDs get two loaders beside the QK wave and the other two a PV
  // pair (split 6: 754 -> 660 us; on grids that fill the chip it cost 1%).
  enum { kRoleQK, kRoleLd, kRolePV };
  template <bool kSpread>
  static __device__ __forceinline__ int role(int w) {
    if (w < kQK) return kRoleQK;
    if (!kSpread) return w < kPVFirst ? kRoleLd : kRolePV;
    return (w & 3) >= 2 && w < 8 ? kRolePV : kRoleLd;
  }
  template <bool kSpread>
  static __device__ __forceinline__ int ld_index(int w) {
    return !kSpread ? w - kLdFirst : (w < 8 ? w - 4 : w - 6);
  }
  template <bool kSpread>
  static __device__ __forceinline__ int pv_index(int w) {
    return !kSpread ? w - kPVFirst : (w < 6 ? w - 2 : w - 4);
  }
};

template <int NT>
struct __attribute__((aligned(16))) BSmem {
  uint8_t pages[kStages][kPageLdsB];
  uint8_t ptile[2][NT * kTileRows * kPRowB];
  float4 cl[2][NT * kTileRows][2];  // per (row, token tile): (c, sum x, sum P~, 0)
};

__device__ __forceinline__ v4i ld16(const uint8_t* base, int off) {
  return *(const v4i*)(base + off);
}

__device__ __forceinline__ v8bf as_bf8(v4i x) { return __builtin_bit_cast(v8bf, x); }

__device__ __forceinline__ void block_sync_lds() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 2^(a - b) for integer-valued a <= b; 0 when a is -inf.
__device__ __forceinline__ float pow2_diff(float a, float b) {
  return a == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(a - b));
}

// Two BF16 values (one 32-bit word) times a power of two; the product of a normal
// BF16 value and a power of two is a BF16 value unless it leaves the normal range.
__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t w, float s) {
  const float lo = __uint_as_float(w << 16) * s;
  const float hi = __uint_as_float(w & 0xFFFF0000u) * s;
  return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

struct BItem {
  const PlanDev* P;
  const uint8_t* q;
  const uint8_t* kv;
  const int32_t* btb;
  float* ws_o;
  float* ws_stats;
  float scale_log2;
  int b, part, L, t0, t1, row0, p_first, p_end, nsteps;  // keys [t0, t1), pages [p_first, p_end)
  int qb;
  int lane, w, g, l16;
};

constexpr int kNoKey = -0x40000000;

template <int NT, bool kSpread, bool kDoQK, bool kDoLd, bool kDoPV>
__device__ __forceinline__ void bwave_main(const BItem& it, BSmem<NT>& sm) {
  static_assert(!kSpread || NT == 1, "spread placement: one row tile");
  using R = BRoles<NT>;
  const PlanDev& P = *it.P;
  const int lane = it.lane, w = it.w, g = it.g, l16 = it.l16;
  const int nsteps = it.nsteps, p_first = it.p_first, p_end = it.p_end, t1 = it.t1, L = it.L;
  const int t0 = it.t0;  // a key window can start inside the first page
  const int row0 = it.row0;

  // ---------------- QK role: (row tile w >> 1, token tile w & 1) ----------------
  const int qk_rt = w >> 1, qk_tt = w & 1;
  constexpr int kQF = kDoQK ? kKSteps : 1;
  v4i qf[kQF];
  int k_base = 0, lim_q = 0, lim_all = 0;
  if (kDoQK) {
    // Q^T fragments: lane (row l16, group g) holds BF16 [32 kk + 8 g, 32 kk + 8 g + 8)
    const int qrow = row0 + qk_rt * kTileRows + l16;
    const bool qrow_valid = qrow < P.rows;
    const uint8_t* qp = it.q + ((int64_t)it.b * P.rows + (qrow_valid ? qrow : 0)) * kRowB;
#pragma unroll
    for (int kk = 0; kk < kQF; ++kk) {
      v4i a = ld16(qp, 64 * kk + 16 * g);
      if (!qrow_valid) a = 0;
      qf[kk] = a;
    }
    const int qb = it.qb;
    const int jq = qrow_valid ? qrow / P.heads : 0;
    lim_q = jq < qb ? min(t1, L - qb + jq + 1) : kNoKey;
    const int j_first = min(row0, P.rows - 1) / P.heads;
    const int j_last = (min(row0 + NT * kTileRows, P.rows) - 1) / P.heads;
    lim_all = j_last >= qb ? kNoKey : min(t1, L - qb + j_first + 1);
    // K operand: token row 16 tt + l16 of the page, BF16 [32 kk + 8 g, ...)
    k_base = (16 * qk_tt + l16) * kRowLdsB + 16 * g;
  }

  auto qk_step = [&](int st) {
    const uint8_t* stage = sm.pages[st % kStages];
    v4f a0 = v4f{0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
    for (int kk = 0; kk < kQF; kk += 2) {
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ld16(stage, k_base + 64 * kk)),
                                                   as_bf8(qf[kk]), a0, 0, 0, 0);
      if (kk + 1 < kQF)
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(ld16(stage, k_base + 64 * kk + 64)),
                                                     as_bf8(qf[kk + 1]), a1, 0, 0, 0);
    }
    // lane holds S[row l16][page token 16 tt + 4 g + jj]
    const int tok_page = (p_first + st) * kPage;
    const bool need_mask = tok_page + kPage > lim_all || tok_page < t0;
    const int tok0 = tok_page + 16 * qk_tt + 4 * g;
    float t[4];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float v = (a0[jj] + a1[jj]) * it.scale_log2;
      if (need_mask && (tok0 + jj >= lim_q || tok0 + jj < t0)) v = -INFINITY;
      t[jj] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float c = ceilf(mx);  // -inf when no key of the tile is visible to the row
    const float off = 8.f - (c == -INFINITY ? 0.f : c);
    float x[4];
    float xs = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      x[jj] = exp2f(t[jj] + off);  // exp2(-inf) = 0
      xs += x[jj];
    }
    __bf16 pb[4];
    float ps = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      pb[jj] = (__bf16)x[jj];
      ps += (float)pb[jj];
    }
    xs += __shfl_xor(xs, 16);
    xs += __shfl_xor(xs, 32);
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, pb[0]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, pb[1]) << 16);
    const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, pb[2]) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, pb[3]) << 16);
    uint8_t* prow = sm.ptile[st & 1] + (qk_rt * kTileRows + l16) * kPRowB + 16 * g + 8 * qk_tt;
    *(uint2*)prow = make_uint2(w0, w1);
    if (g == 0) sm.cl[st & 1][qk_rt * kTileRows + l16][qk_tt] = make_float4(c, xs, ps, 0.f);
  };

  // ---------------- loader role ----------------
  const int li = R::template ld_index<kSpread>(w);
  constexpr int kLd = kDoLd ? R::kMaxLd : 1;
  // Loader li owns the kLd consecutive 1 KB chunks li kLd .. li kLd + kLd - 1 of the
  // step's page; lane i moves 16 bytes into padded LDS row n.
  const uint32_t ld_byte0 = (uint32_t)(max(li, 0) * kLd * 1024 + 16 * lane);
  // steps past the split's end repeat its last page (loads without conditions whose
  // data is never read)
  auto page_id = [&](int st) -> int64_t { return it.btb[min(p_first + st, p_end - 1)]; };
  auto gload = [&](int64_t id, v4i (&buf)[kLd]) {
    const uint8_t* gp = it.kv + id * kPageB + ld_byte0;
#pragma unroll
    for (int i = 0; i < kLd; ++i) buf[i] = __builtin_nontemporal_load((const v4i*)(gp + 1024 * i));
  };
  auto lstore = [&](int st, const v4i (&buf)[kLd]) {
    uint8_t* stage = sm.pages[st % kStages];
    uint32_t b0 = ld_byte0;
    __asm__ volatile("" : "+v"(b0));
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const uint32_t byte = b0 + 1024 * i;
      const uint32_t n = byte / kRowB;
      *(v4i*)(stage + byte + (kRowLdsB - kRowB) * n) = buf[i];
    }
  };

  // ---------------- PV role ----------------
  const int pv_w = R::template pv_index<kSpread>(w);
  constexpr int kDT = kDoPV ? R::kDimTiles : 1;
  constexpr int kNTp = kDoPV ? NT : 1;
  v4f acc[kNTp][kDT];
  float m_c[kNTp][4];  // running max of result rows 4 g + jj
  float m_a[kNTp];     // running max of operand row l16
  float lsum[4] = {0.f, 0.f, 0.f, 0.f}, ltil[4] = {0.f, 0.f, 0.f, 0.f};  // row tile pv_w
#pragma unroll
  for (int rt = 0; rt < kNTp; ++rt) {
    m_a[rt] = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) m_c[rt][jj] = -INFINITY;
#pragma unroll
    for (int d = 0; d < kDT; ++d) acc[rt][d] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // transposed V reads: lane (16 G + u), read r addresses token 16 r + 4 G + u / 4 and
  // dims 16 D + 4 (u % 4) .. + 3; lane 16 G + u receives dim 16 D + u of tokens
  // 16 r + 4 G .. 16 r + 4 G + 3.
  int tr_base[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    tr_base[r] = (16 * r + 4 * g + (l16 >> 2)) * kRowLdsB + 32 * R::kDimTiles * max(pv_w, 0) +
                 8 * (l16 & 3);

  auto pv_step = [&](int st) {
    const uint8_t* stage = sm.pages[st % kStages];
    const int pb = st & 1;
    v8bf pa[kNTp];
#pragma unroll
    for (int rt = 0; rt < kNTp; ++rt) {
      bool rescale = false;
      float alpha[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 p0 = sm.cl[pb][rt * kTileRows + 4 * g + jj][0];
        const float4 p1 = sm.cl[pb][rt * kTileRows + 4 * g + jj][1];
        const float mn = fmaxf(m_c[rt][jj], fmaxf(p0.x, p1.x));
        alpha[jj] = mn == m_c[rt][jj] ? 1.f : pow2_diff(m_c[rt][jj], mn);
        rescale |= mn != m_c[rt][jj];
        if (rt == pv_w) {
          const float w0 = pow2_diff(p0.x, mn), w1 = pow2_diff(p1.x, mn);
          lsum[jj] = lsum[jj] * alpha[jj] + p0.y * w0 + p1.y * w1;
          ltil[jj] = ltil[jj] * alpha[jj] + p0.z * w0 + p1.z * w1;
        }
        m_c[rt][jj] = mn;
      }
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
        for (int d = 0; d < kDT; ++d) {
          acc[rt][d][0] *= alpha[0]; acc[rt][d][1] *= alpha[1];
          acc[rt][d][2] *= alpha[2]; acc[rt][d][3] *= alpha[3];
        }
      }
      // operand row l16: tile tt's P~ times 2^(c_tt - m)
      const float4 a0 = sm.cl[pb][rt * kTileRows + l16][0];
      const float4 a1 = sm.cl[pb][rt * kTileRows + l16][1];
      m_a[rt] = fmaxf(m_a[rt], fmaxf(a0.x, a1.x));
      const float s0 = pow2_diff(a0.x, m_a[rt]), s1 = pow2_diff(a1.x, m_a[rt]);
      v4i pw = ld16(sm.ptile[pb], (rt * kTileRows + l16) * kPRowB + 16 * g);
      if (__builtin_amdgcn_ballot_w64(s0 != 1.f || s1 != 1.f) != 0) {
        pw.x = (int)scale_bf16x2((uint32_t)pw.x, s0);
        pw.y = (int)scale_bf16x2((uint32_t)pw.y, s0);
        pw.z = (int)scale_bf16x2((uint32_t)pw.z, s1);
        pw.w = (int)scale_bf16x2((uint32_t)pw.w, s1);
      }
      pa[rt] = as_bf8(pw);
    }
    // tokens past the split's end, or before a window's start in the first page, may
    // hold poison: zero their V elements (P~ is 0)
    uint32_t mk[2][2] = {{0xFFFFFFFFu, 0xFFFFFFFFu}, {0xFFFFFFFFu, 0xFFFFFFFFu}};
    if (st == nsteps - 1 || (st == 0 && t0 > p_first * kPage)) {
      const int valid = t1 - (p_first + st) * kPage;
      const int skip = st == 0 ? t0 - p_first * kPage : 0;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tk = 16 * r + 4 * g + 2 * h;
          mk[r][h] = (tk < valid && tk >= skip ? 0x0000FFFFu : 0u) |
                     (tk + 1 < valid && tk + 1 >= skip ? 0xFFFF0000u : 0u);
        }
    }
#pragma unroll
    for (int d = 0; d < kDT; ++d) {
      const v4s b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(stage + tr_base[0] + 32 * d));
      const v4s b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(stage + tr_base[1] + 32 * d));
      const v2u x0 = __builtin_bit_cast(v2u, b0);
      const v2u x1 = __builtin_bit_cast(v2u, b1);
      const v4i vb = v4i{(int)(x0.x & mk[0][0]), (int)(x0.y & mk[0][1]),
                         (int)(x1.x & mk[1][0]), (int)(x1.y & mk[1][1])};
#pragma unroll
      for (int rt = 0; rt < kNTp; ++rt)
        acc[rt][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[rt], as_bf8(vb), acc[rt][d], 0, 0, 0);
    }
  };

  // ---------------- pipeline (as the FP8 kernel, one page per step) ----------------
  v4i bufA[kLd], bufB[kLd];
  int64_t nid = 0;
  if (kDoLd && nsteps > 0) {
    gload(page_id(0), bufA);
    gload(page_id(1), bufB);
    lstore(0, bufA);
    gload(page_id(2), bufA);
    lstore(1, bufB);
    gload(page_id(3), bufB);
    nid = page_id(4);
  }
  block_sync_lds();  // steps 0 and 1 stored
  if (kDoQK && nsteps > 0) qk_step(0);
  const int npairs = nsteps >> 1;
  for (int i = 0; i < npairs; ++i) {
    const int st = 2 * i;
    block_sync_lds();  // stage st + 1 stored, P~(st) ready, PV(st - 1) done everywhere
    if (kDoLd) {
      lstore(st + 2, bufA);
      gload(nid, bufA);
      nid = page_id(st + 5);
    }
    if (kDoQK) qk_step(st + 1);
    if (kDoPV) pv_step(st);
    block_sync_lds();
    if (kDoLd) {
      lstore(st + 3, bufB);
      gload(nid, bufB);
      nid = page_id(st + 6);
    }
    if (kDoQK && st + 2 < nsteps) qk_step(st + 2);
    if (kDoPV) pv_step(st + 1);
  }
  if (nsteps & 1) {
    block_sync_lds();
    if (kDoPV) pv_step(nsteps - 1);
  }

  // ---------------- write the partials ----------------
  if (kDoPV) {
    const int64_t part_row0 = (int64_t)it.part * P.rows;
#pragma unroll
    for (int rt = 0; rt < kNTp; ++rt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int row = row0 + rt * kTileRows + 4 * g + jj;
        if (row < P.rows) {
          float* orow = it.ws_o + (part_row0 + row) * kDV + 16 * R::kDimTiles * pv_w + l16;
#pragma unroll
          for (int d = 0; d < kDT; ++d) orow[16 * d] = acc[rt][d][jj];
          if (rt == pv_w && l16 == 0)
            *(float4*)(it.ws_stats + (part_row0 + row) * kStatStride) =
                make_float4(m_c[rt][jj], lsum[jj], ltil[jj], 0.f);
        }
      }
    }
  }
}

template <int NT, bool kDev, bool kSpread>
__global__ void __launch_bounds__(BRoles<NT>::kThreads, 1)
partial_bf16_kernel(const PlanDev Parg, const PlanDev* __restrict__ pdev,
                    const float* __restrict__ scale_dev, const uint8_t* __restrict__ q,
                    const uint8_t* __restrict__ kv, const int32_t* __restrict__ bt,
                    int64_t bt_stride, const int32_t* __restrict__ kv_lens,
                    const int32_t* __restrict__ q_lens, const int32_t* __restrict__ kv_bounds,
                    float scale_log2_arg, float* __restrict__ ws_o, float* __restrict__ ws_stats) {
  __shared__ BSmem<NT> sm;
  const PlanDev& P = kDev ? *pdev : Parg;
  const float scale_log2 = kDev ? *scale_dev * 1.4426950408889634f : scale_log2_arg;
  BItem it;
  it.lane = threadIdx.x & 63;
  it.w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
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
  it.nsteps = it.t1 > it.t0 ? it.p_end - it.p_first : 0;

  const int w = it.w;
  using R = BRoles<NT>;
  const int role = R::template role<kSpread>(w);
  if (role == R::kRoleQK) bwave_main<NT, kSpread, true, false, false>(it, sm);
  else if (role == R::kRoleLd) bwave_main<NT, kSpread, false, true, false>(it, sm);
  else bwave_main<NT, kSpread, false, false, true>(it, sm);
}

}  // namespace

int launch_partial_bf16(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                        const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                        float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                        const DeviceArgs* dev, const int32_t* q_lens, const int32_t* kv_bounds) {
  const PlanDev& P = plan.dev;
  const int slots = (P.total_parts * P.subs + 7) / 8;
  const dim3 grid(8 * slots * P.tiles);
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const PlanDev* pd = dev ? dev->plan : nullptr;
  const float* sd = dev ? dev->softmax_scale : nullptr;
  hipStream_t st = (hipStream_t)stream;
#define MLA_BF16_LAUNCH(NT, DEV, SPREAD)                                                    \
  hipLaunchKernelGGL((partial_bf16_kernel<NT, DEV, SPREAD>), grid, dim3(BRoles<NT>::kThreads), \
                     0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds,       \
                     scale_log2, ws_o, ws_stats)
  if (P.nt == 1 && narrow_underfilled(plan)) {
    if (dev) MLA_BF16_LAUNCH(1, true, true); else MLA_BF16_LAUNCH(1, false, true);
  } else if (P.nt == 1) {
    if (dev) MLA_BF16_LAUNCH(1, true, false); else MLA_BF16_LAUNCH(1, false, false);
  } else {
    if (dev) MLA_BF16_LAUNCH(2, true, false); else MLA_BF16_LAUNCH(2, false, false);
  }
#undef MLA_BF16_LAUNCH
  return (int)hipGetLastError();
}

}  // namespace mla
