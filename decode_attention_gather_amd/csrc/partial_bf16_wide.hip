// Split-KV partial kernel for MLA decode over a paged BF16 cache, wide row blocks (64
// or 96 query rows), gfx950.
//
// The BF16 variant that TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower after
// #19338" measures beside the FP8 kernel (Repro 2), for requests of more than 32 query
// rows (q = 8, many heads). It computes exactly what partial_bf16.hip computes, per
// (request b, split s, block of 16 NT query rows, NT = 4 or 6): the state of PR #20380 "trtllm-gen
// FMHA: split the KV partials of a row across thread groups in fmhaReductionKernel"
// (Description: per-row max, sum and unnormalised O) with P~ the BF16 rounding of
// 2^(t - c + 8) per 16-token tile, scaled by 2^(c - m) before the PV product. Here one
// staged page feeds up to 96 rows, so a page crosses HBM -> LDS once per 96 rows
// instead of once per 32.
//
// Design for gfx950: one workgroup of NT/2 + 4 wavefronts per work item (at most 2 per
// SIMD, so every wave may hold 256 VGPRs).
//  * Gather: direct-to-LDS loads (global_load_lds_dwordx4, 1 KB per instruction) of one
//    page (36 KB) per pipeline step into a 3-stage ring, issued by the PV waves two
//    steps ahead. Rows stay 1152 bytes; 16-byte chunk c of token row n sits at chunk
//    (c + ((n >> 1) & 7)) mod 72, which puts the 16 rows of an operand read on distinct
//    LDS banks (a row is 288 dwords, so consecutive rows start half of the 64 banks
//    apart, and the rotation spreads 8 row pairs over the other half-offsets).
//  * QK^T: NT/2 QK waves; wave q holds Q^T of row tiles 2q, 2q + 1 (144 VGPRs: BF16
//    Q^T of three tiles would not fit beside the accumulators) and forms S^T = K Q^T of
//    both 16-token tiles of the page on v_mfma_f32_16x16x32_bf16; every K fragment
//    read feeds two MFMAs. Softmax per (row, tile): c = ceil(max t),
//    x = 2^(t - c + 8), P~ = BF16(x) to LDS with c; the QK waves also keep each row's
//    running maximum m and l = sum x, l~ = sum P~ (both scaled to m).
//  * PV: 4 waves; wave (group pg, half dh) keeps the running maximum m of row tiles
//    [pg NT/2, (pg + 1) NT/2), scales their P~ rows by 2^(c - m) (exact), and
//    accumulates O for dims [256 dh, 256 dh + 256) with V gathered transposed by
//    ds_read_b64_tr_b16; each V read feeds NT/2 MFMAs. With 3 QK waves beside 4 PV
//    waves (NT = 6) every SIMD but one runs one QK and one PV wave. K position 8 G + 4 tt + j of an MFMA (G = lane group) holds
//    token 16 tt + 4 G + j, where both the QK results and the transposed reads put it.
//  * Skewed single-barrier pipeline: iteration s runs QK/softmax of step s + 1 and PV of
//    step s; P~ and the tile statistics are double-buffered.
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
constexpr int kPageB = kPage * kRowB;               // 36864 bytes per page
constexpr int kStages = 3;
constexpr int kChunks = kRowB / 16;                 // 72 chunks of 16 bytes per row
constexpr int kLoads = kPageB / 1024;               // 36 wave-wide 16-byte loads per page
constexpr int kKSteps = kDQK / 32;                  // 18 MFMAs of K = 32 per 576-wide dot
constexpr int kPRowB = 80;                          // P~ row: 32 BF16 + 16 bytes of pad

// Roles: NT/2 QK waves, wave q holding Q^T of row tiles 2 q, 2 q + 1; 4 PV waves,
// wave (group pg, half dh) accumulating O of row tiles [pg NT/2, (pg + 1) NT/2) and
// dims [256 dh, 256 dh + 256), and issuing 9 of the step's 36 direct-to-LDS loads.
template <int NT>
struct BWRoles {
  static_assert(NT == 4 || NT == 6, "wide row blocks hold 4 or 6 row tiles");
  static constexpr int kQKW = NT / 2;
  static constexpr int kQKT = 2;                     // row tiles per QK wave
  static constexpr int kPVW = 4;
  static constexpr int kPVT = NT / 2;                // row tiles per PV wave
  static constexpr int kWaves = kQKW + kPVW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kDMA = kLoads / kPVW;         // 9 loads per PV wave per step
  static_assert(kDMA * kPVW == kLoads && kWaves <= 8, "roles");
};

template <int NT>
struct __attribute__((aligned(16))) BWSmem {
  uint8_t pages[kStages][kPageB];
  uint8_t ptile[2][NT * kTileRows * kPRowB];
  float2 cl[2][NT * kTileRows];  // per row: c of token tiles 0 and 1
};

__device__ __forceinline__ int rot_of(int n) { return (n >> 1) & 7; }

__device__ __forceinline__ v4i ld16(const uint8_t* base, int off) {
  return *(const v4i*)(base + off);
}

__device__ __forceinline__ v8bf as_bf8(v4i x) { return __builtin_bit_cast(v8bf, x); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void block_sync_lds() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wave-wide direct-to-LDS load (lane i's 16 bytes at sbase + voff land at LDS byte
// lds_base + 16 i), from inline asm so that the compiler's wait counts do not drain it
// at every LDS access; M0 carries the LDS base and is restored; the s_nop covers the
// wait states after a VALU write of an SGPR the load reads.
__device__ __forceinline__ void dma16(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(base)
      : "memory");
}

__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

__device__ __forceinline__ float group_max4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 2^(a - b) for integer-valued a <= b; 0 when a is -inf.
__device__ __forceinline__ float pow2_diff(float a, float b) {
  return a == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(a - b));
}

// Two BF16 values (one 32-bit word) times a power of two (exact for normal values).
__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t w, float s) {
  const float lo = __uint_as_float(w << 16) * s;
  const float hi = __uint_as_float(w & 0xFFFF0000u) * s;
  return (__float_as_uint(hi) & 0xFFFF0000u) | (__float_as_uint(lo) >> 16);
}

__device__ __forceinline__ bool wg_item(const PlanDev& P, int wg, int* part_sorted, int* blk) {
  const int x = wg & 7, k = wg >> 3;
  const int slot = k / P.tiles;
  *blk = k - slot * P.tiles;
  *part_sorted = slot * 8 + x;
  return *part_sorted < P.total_parts;
}

struct BWItem {
  const PlanDev* P;
  const uint8_t* q;
  const uint8_t* kv;
  const int32_t* btb;
  float* ws_o;
  float* ws_stats;
  float scale_log2;
  int b, part, L, t1, row0, p_first, p_end, nsteps;
  int qb;
  int lane, w, g, l16;
};

constexpr int kNoKey = -0x40000000;

// ------------------------------------------------------------------ QK waves
template <int NT>
__device__ __forceinline__ void bw_qk(const BWItem& it, BWSmem<NT>& sm) {
  using R = BWRoles<NT>;
  constexpr int kQKT = R::kQKT, kCh = 2;  // two accumulator chains per row tile
  const PlanDev& P = *it.P;
  const int g = it.g, l16 = it.l16, qw = it.w;
  const int nsteps = it.nsteps, p_first = it.p_first, t1 = it.t1;

  // Q^T fragments of row tiles 2 qw + k: lane (row l16, group g) holds BF16
  // [32 kk + 8 g, 32 kk + 8 g + 8) of its row
  v4i qf[kQKT][kKSteps];
  int lim_q[kQKT];
#pragma unroll
  for (int k = 0; k < kQKT; ++k) {
    const int qrow = it.row0 + (qw * kQKT + k) * kTileRows + l16;
    const bool valid = qrow < P.rows;
    const uint8_t* qp = it.q + ((int64_t)it.b * P.rows + (valid ? qrow : 0)) * kRowB;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      v4i a = ld16(qp, 64 * kk + 16 * g);
      if (!valid) a = 0;
      qf[k][kk] = a;
    }
    const int jq = valid ? qrow / P.heads : 0;
    lim_q[k] = jq < it.qb ? min(t1, it.L - it.qb + jq + 1) : kNoKey;
  }
  const int first_row = min(it.row0 + qw * kQKT * kTileRows, P.rows - 1);
  const int last_row = min(it.row0 + (qw + 1) * kQKT * kTileRows, P.rows) - 1;
  const int lim_all = last_row / P.heads >= it.qb
      ? kNoKey : min(t1, it.L - it.qb + first_row / P.heads + 1);

  // running maximum and sums of row l16 of tile k (the same in the four lane groups)
  float m_run[kQKT], l_run[kQKT], lt_run[kQKT];
#pragma unroll
  for (int k = 0; k < kQKT; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = lt_run[k] = 0.f;
  }

  // K operand of token row n = 16 tt + l16: chunk 4 kk + g at (4 kk + g + rot(n)) mod 72;
  // rot(n) = (l16 >> 1) & 7 for both tiles. Latent steps (kk < 16) never wrap.
  const int rot = rot_of(l16);
  const int k_lat = 16 * (g + rot);
  int k_rope[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) k_rope[r] = 16 * ((64 + 4 * r + g + rot) % kChunks);

  auto qk_step = [&](int st) {
    const uint8_t* stage = sm.pages[st % kStages];
    const int tok_page = (p_first + st) * kPage;
    const bool need_mask = tok_page + kPage > lim_all;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint8_t* rowp = stage + (16 * tt + l16) * kRowB;
      v4f acc[kQKT][kCh];
#pragma unroll
      for (int k = 0; k < kQKT; ++k)
#pragma unroll
        for (int c = 0; c < kCh; ++c) acc[k][c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKSteps; ++kk) {
        const int off = kk < 16 ? k_lat + 64 * kk : k_rope[kk - 16];
        const v8bf kf = as_bf8(ld16(rowp, off));
#pragma unroll
        for (int k = 0; k < kQKT; ++k)
          acc[k][kk % kCh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, as_bf8(qf[k][kk]), acc[k][kk % kCh], 0, 0, 0);
      }
      // lane holds S[row l16][page token 16 tt + 4 g + jj]
      const int tok0 = tok_page + 16 * tt + 4 * g;
#pragma unroll
      for (int k = 0; k < kQKT; ++k) {
        float t[4];
        float mx = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float v = (acc[k][0][jj] + acc[k][1][jj]) * it.scale_log2;
          if (need_mask && tok0 + jj >= lim_q[k]) v = -INFINITY;
          t[jj] = v;
          mx = fmaxf(mx, v);
        }
        mx = group_max4(mx);
        const float c = ceilf(mx);  // -inf when no key of the tile is visible to the row
        const float off = 8.f - (c == -INFINITY ? 0.f : c);
        float xs = 0.f, ps = 0.f;
        uint32_t pw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float x0 = __builtin_amdgcn_exp2f(t[2 * h] + off);  // exp2(-inf) = 0
          const float x1 = __builtin_amdgcn_exp2f(t[2 * h + 1] + off);
          xs += x0 + x1;
          const __bf16 b0 = (__bf16)x0, b1 = (__bf16)x1;
          ps += (float)b0 + (float)b1;
          pw[h] = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                  ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        }
        xs = group_sum4(xs);
        ps = group_sum4(ps);
        const int row = (qw * kQKT + k) * kTileRows + l16;
        *(uint2*)(sm.ptile[st & 1] + row * kPRowB + 16 * g + 8 * tt) = make_uint2(pw[0], pw[1]);
        if (g == 0) ((float*)&sm.cl[st & 1][row])[tt] = c;
        const float mn = fmaxf(m_run[k], c);
        const float a = pow2_diff(m_run[k], mn), wt = pow2_diff(c, mn);
        l_run[k] = l_run[k] * a + xs * wt;
        lt_run[k] = lt_run[k] * a + ps * wt;
        m_run[k] = mn;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __builtin_amdgcn_s_setprio(2);  // the QK waves pace the step: issue first on their SIMD
  block_sync_lds();               // step 0 landed
  if (nsteps > 0) qk_step(0);
  for (int st = 0; st < nsteps; ++st) {
    block_sync_lds();
    if (st + 1 < nsteps) qk_step(st + 1);
  }

  // (m, l, l~) of rows 2 qw 16 + 16 k + l16; m is the maximum the PV waves scale O to
  if (g == 0) {
    const int64_t part_row0 = (int64_t)it.part * P.rows;
#pragma unroll
    for (int k = 0; k < kQKT; ++k) {
      const int row = it.row0 + (qw * kQKT + k) * kTileRows + l16;
      if (row < P.rows)
        *(float4*)(it.ws_stats + (part_row0 + row) * kStatStride) =
            make_float4(m_run[k], l_run[k], lt_run[k], 0.f);
    }
  }
}

// ------------------------------------------------------------------ PV waves
template <int NT>
__device__ __forceinline__ void bw_pv(const BWItem& it, BWSmem<NT>& sm) {
  using R = BWRoles<NT>;
  constexpr int kRT = R::kPVT;  // row tiles per PV wave
  constexpr int kDT = 16;          // 16-dim tiles per PV wave
  constexpr int kDMA = R::kDMA;
  const PlanDev& P = *it.P;
  const int g = it.g, l16 = it.l16, lane = it.lane;
  const int nsteps = it.nsteps, p_first = it.p_first, p_end = it.p_end, t1 = it.t1;
  const int pv = it.w - R::kQKW;
  const int rt0 = (pv >> 1) * kRT;  // group pv >> 1
  const int dh = pv & 1;

  // Direct-to-LDS loads k = pv kDMA + i of a step: LDS bytes [1024 k, 1024 k + 1024) of
  // the stage; lane i fills 16-byte slot s = 64 k + i, which holds chunk
  // (s % 72 - rot(s / 72)) mod 72 of token row s / 72. Offsets are recomputed at each
  // issue (the asm keeps the compiler from keeping them live across the loop).
  auto src_off = [&](int k) -> uint32_t {
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    const int slot = k * 64 + ln;
    const int n = slot / kChunks, pos = slot - n * kChunks;
    int c = pos - rot_of(n);
    if (c < 0) c += kChunks;
    return (uint32_t)(n * kRowB + 16 * c);
  };
  auto issue = [&](int st, int64_t id) {
    const uint64_t gp = uniform_addr(it.kv + id * kPageB);
    uint8_t* stage = sm.pages[st % kStages];
#pragma unroll
    for (int i = 0; i < kDMA; ++i) {
      const int k = pv * kDMA + i;
      dma16(gp, src_off(k), (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(stage + k * 1024));
    }
  };
  auto page_id = [&](int st) -> int64_t { return it.btb[min(p_first + st, p_end - 1)]; };

  v4f acc[kRT][kDT];
  float m_c[kRT][4];  // running max of result rows 4 g + jj
  float m_a[kRT];     // running max of operand row l16
#pragma unroll
  for (int k = 0; k < kRT; ++k) {
    m_a[k] = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) m_c[k][jj] = -INFINITY;
#pragma unroll
    for (int d = 0; d < kDT; ++d) acc[k][d] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  // transposed V reads: lane (16 G + u), read r addresses token 16 r + 4 G + u / 4 and
  // dims 16 D + 4 (u % 4) .. + 3 (chunk 2 D + (u % 4) / 2, rotated, never wrapping);
  // lane 16 G + u receives dim 16 D + u of tokens 16 r + 4 G .. 16 r + 4 G + 3
  int tr_base[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 16 * r + 4 * g + (l16 >> 2);
    tr_base[r] = t * kRowB + 16 * (((l16 & 3) >> 1) + rot_of(t)) + 8 * (l16 & 1) + 512 * dh;
  }

  auto pv_step = [&](int st) {
    const uint8_t* stage = sm.pages[st % kStages];
    const int pb = st & 1;
    v8bf pa[kRT];
#pragma unroll
    for (int k = 0; k < kRT; ++k) {
      const int rt = rt0 + k;
      bool rescale = false;
      float alpha[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float2 cc = sm.cl[pb][rt * kTileRows + 4 * g + jj];
        const float mn = fmaxf(m_c[k][jj], fmaxf(cc.x, cc.y));
        alpha[jj] = mn == m_c[k][jj] ? 1.f : pow2_diff(m_c[k][jj], mn);
        rescale |= mn != m_c[k][jj];
        m_c[k][jj] = mn;
      }
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
        for (int d = 0; d < kDT; ++d) {
          acc[k][d][0] *= alpha[0]; acc[k][d][1] *= alpha[1];
          acc[k][d][2] *= alpha[2]; acc[k][d][3] *= alpha[3];
        }
      }
      // operand row l16: tile tt's P~ times 2^(c_tt - m)
      const float2 ca = sm.cl[pb][rt * kTileRows + l16];
      m_a[k] = fmaxf(m_a[k], fmaxf(ca.x, ca.y));
      const float s0 = pow2_diff(ca.x, m_a[k]), s1 = pow2_diff(ca.y, m_a[k]);
      v4i pw = ld16(sm.ptile[pb], (rt * kTileRows + l16) * kPRowB + 16 * g);
      if (__builtin_amdgcn_ballot_w64(s0 != 1.f || s1 != 1.f) != 0) {
        pw.x = (int)scale_bf16x2((uint32_t)pw.x, s0);
        pw.y = (int)scale_bf16x2((uint32_t)pw.y, s0);
        pw.z = (int)scale_bf16x2((uint32_t)pw.z, s1);
        pw.w = (int)scale_bf16x2((uint32_t)pw.w, s1);
      }
      pa[k] = as_bf8(pw);
    }
    // tokens past the split's end may hold poison: zero their V elements (P~ is 0)
    uint32_t mk[2][2] = {{0xFFFFFFFFu, 0xFFFFFFFFu}, {0xFFFFFFFFu, 0xFFFFFFFFu}};
    if (st == nsteps - 1) {
      const int valid = t1 - (p_first + st) * kPage;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int tk = 16 * r + 4 * g + 2 * h;
          mk[r][h] = (tk < valid ? 0x0000FFFFu : 0u) | (tk + 1 < valid ? 0xFFFF0000u : 0u);
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
      for (int k = 0; k < kRT; ++k)
        acc[k][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[k], as_bf8(vb), acc[k][d], 0, 0, 0);
    }
  };

  // ---- pipeline: 1 + nsteps barriers, like the QK waves; a step's page id is read one
  // step before its loads are issued
  int64_t nid = 0;
  if (nsteps > 0) issue(0, page_id(0));
  if (nsteps > 1) issue(1, page_id(1));
  if (nsteps > 2) nid = page_id(2);
  if (nsteps > 1) wait_vmcnt<kDMA>(); else wait_vmcnt<0>();  // step 0 landed
  block_sync_lds();
  for (int st = 0; st < nsteps; ++st) {
    wait_vmcnt<0>();  // step st + 1 landed
    block_sync_lds();
    if (st + 2 < nsteps) {
      issue(st + 2, nid);
      if (st + 3 < nsteps) nid = page_id(st + 3);
    }
    pv_step(st);
  }

  // ---- partials: O rows rt 16 + 4 g + jj, dims 256 dh + 16 d + l16
  const int64_t part_row0 = (int64_t)it.part * P.rows;
#pragma unroll
  for (int k = 0; k < kRT; ++k) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = it.row0 + (rt0 + k) * kTileRows + 4 * g + jj;
      if (row < P.rows) {
        float* orow = it.ws_o + (part_row0 + row) * kDV + 256 * dh + l16;
#pragma unroll
        for (int d = 0; d < kDT; ++d) orow[16 * d] = acc[k][d][jj];
      }
    }
  }
}

template <int NT, bool kDev>
__global__ void __launch_bounds__(BWRoles<NT>::kThreads, 1)
partial_bf16_wide_kernel(const PlanDev Parg, const PlanDev* __restrict__ pdev,
                         const float* __restrict__ scale_dev, const uint8_t* __restrict__ q,
                         const uint8_t* __restrict__ kv, const int32_t* __restrict__ bt,
                         int64_t bt_stride, const int32_t* __restrict__ kv_lens,
                         const int32_t* __restrict__ q_lens, float scale_log2_arg,
                         float* __restrict__ ws_o, float* __restrict__ ws_stats) {
  __shared__ BWSmem<NT> sm;
  const PlanDev& P = kDev ? *pdev : Parg;
  const float scale_log2 = kDev ? *scale_dev * 1.4426950408889634f : scale_log2_arg;
  BWItem it;
  it.lane = threadIdx.x & 63;
  it.w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  it.g = it.lane >> 4;
  it.l16 = it.lane & 15;
  int ps, blk;
  if (!wg_item(P, blockIdx.x, &ps, &blk)) return;
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
  it.part = (int)P.part_base[b] + s;
  it.L = min(kv_lens[b], (int)P.kv_len[b]);
  it.qb = q_lens != nullptr ? min(max(q_lens[b], 0), P.q_len) : P.q_len;
  const int chunk_tok = chunk_pages_of(P, b) * kPage;
  const int t0 = s * chunk_tok;
  it.t1 = max(t0, min(t0 + chunk_tok, it.L));
  it.row0 = blk * NT * kTileRows;
  it.p_first = t0 / kPage;
  it.p_end = (it.t1 + kPage - 1) / kPage;
  it.nsteps = it.t1 > t0 ? it.p_end - it.p_first : 0;

  if (it.w < BWRoles<NT>::kQKW) bw_qk<NT>(it, sm);
  else bw_pv<NT>(it, sm);
}

}  // namespace

int launch_partial_bf16_wide(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                             const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                             float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                             const DeviceArgs* dev, const int32_t* q_lens) {
  const PlanDev& P = plan.dev;
  const int slots = (P.total_parts + 7) / 8;
  const dim3 grid(8 * slots * P.tiles);
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const PlanDev* pd = dev ? dev->plan : nullptr;
  const float* sd = dev ? dev->softmax_scale : nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (P.nt == 4) {
    const dim3 block(BWRoles<4>::kThreads);
    if (dev)
      hipLaunchKernelGGL((partial_bf16_wide_kernel<4, true>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, scale_log2, ws_o, ws_stats);
    else
      hipLaunchKernelGGL((partial_bf16_wide_kernel<4, false>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, scale_log2, ws_o, ws_stats);
  } else {
    const dim3 block(BWRoles<6>::kThreads);
    if (dev)
      hipLaunchKernelGGL((partial_bf16_wide_kernel<6, true>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, scale_log2, ws_o, ws_stats);
    else
      hipLaunchKernelGGL((partial_bf16_wide_kernel<6, false>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, scale_log2, ws_o, ws_stats);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
