// Split-KV partial kernel for MLA decode over a paged BF16 cache, wide row blocks (64
// or 96 query rows), gfx950.
//
// The BF16 variant that TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower after
// #19338" measures beside the FP8 kernel (Repro 2), for requests of more than 32 query
// rows (q = 8, many heads). Per (request b, split s, block of 16 NT query rows, NT = 4
// or 6) it writes the state of PR #20380 "trtllm-gen FMHA: split the KV partials of a
// row across thread groups in fmhaReductionKernel" (Description: per-row max, sum and
// unnormalised O) as partial_bf16.hip does: P~ is the BF16 rounding of 2^(t - c + 8)
// per 16-token tile (c = ceil of the tile's max), times 2^(c - m) with m the running
// maximum. Here the QK waves form that product before they publish P~: rounding
// commutes with a power-of-two scale, so the bits are the same wherever P~ is a normal
// BF16 value (the rest lies more than 2^126 below the row's largest term). One staged
// page feeds up to 96 rows, so a page crosses HBM -> LDS once per 96 rows instead of
// once per 32.
//
// Design for gfx950: one workgroup of NT/2 + 4 wavefronts per work item (at most 2 per
// SIMD, so every wave may hold 256 VGPRs).
//  * Gather: direct-to-LDS loads (global_load_lds_dwordx4, 1 KB per instruction) of one
//    page (36 KB) per pipeline step into a 4-stage ring (160 KB of LDS with P~), issued
//    by the PV waves three steps ahead between their MFMAs, so a load has two steps to
//    land. Rows stay 1152 bytes; 16-byte chunk c of token row n sits at chunk
//    (c + rot(n)) mod 72 with rot(n) = 2 ((n >> 1) & 3) + ((n >> 3) & 1). A row is 288
//    dwords, so consecutive rows start half of the 64 banks apart; the rotation then
//    puts the 16 rows of a K operand read (16 bytes per lane) on 16 distinct 4-bank
//    groups, and the 8 tokens that one pass of a transposed V read serves (32 bytes
//    each) on 8 distinct 8-bank groups. Rows past the split's end are zeroed in LDS
//    once, so V needs no mask.
//  * QK^T: NT/2 QK waves; wave q holds Q^T of row tiles 2q, 2q + 1 (144 VGPRs: BF16
//    Q^T of three tiles would not fit beside the accumulators) and forms S^T = K Q^T of
//    both 16-token tiles of the page on v_mfma_f32_16x16x32_bf16, K fragments read two
//    steps of the dot product ahead; every K fragment feeds two MFMAs. Softmax per row:
//    c per tile, the new running maximum m, x = 2^(t - c + 8), P~ = BF16(x 2^(c - m))
//    to LDS with the rescale factor 2^(m_old - m) of the row; l = sum x and l~ = sum P~
//    (both scaled to m) stay in the QK waves.
//  * PV: 4 waves; wave (group pg, half dh) accumulates O of row tiles
//    [pg NT/2, (pg + 1) NT/2) for dims [256 dh, 256 dh + 256), rescaling it when a row's
//    maximum moved, with V gathered transposed by ds_read_b64_tr_b16 two dim tiles
//    ahead; each V read feeds NT/2 MFMAs. With 3 QK waves beside 4 PV waves (NT = 6)
//    every SIMD but one runs one QK and one PV wave. K position 8 G + 4 tt + j of an
//    MFMA (G = lane group) holds token 16 tt + 4 G + j, where both the QK results and
//    the transposed reads put it.
//  * Skewed single-barrier pipeline: iteration s runs QK/softmax of step s + 1 and PV of
//    step s; P~ and the rescale factors are double-buffered.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "mla_internal.h"

namespace mla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kRowB = 2 * kDQK;                     // 1152 bytes per token row
constexpr int kPageB = kPage * kRowB;               // 36864 bytes per page
constexpr int kStages = 4;
constexpr int kChunks = kRowB / 16;                 // 72 chunks of 16 bytes per row
constexpr int kLoads = kPageB / 1024;               // 36 wave-wide 16-byte loads per page
constexpr int kKSteps = kDQK / 32;                  // 18 MFMAs of K = 32 per 576-wide dot
constexpr int kPRowB = 64;                          // P~ row: 32 BF16

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
  uint8_t ptile[2][NT * kTileRows * kPRowB];  // P~, scaled to the running maximum
  float alpha[2][NT * kTileRows];             // per row: 2^(m_old - m_new) of the step
};

// Chunk rotation of token row n (see the layout note at the top).
__device__ __forceinline__ int rot_of(int n) { return 2 * ((n >> 1) & 3) + ((n >> 3) & 1); }

__device__ __forceinline__ v4i ld16(const uint8_t* base, int off) {
  return *(const v4i*)(base + off);
}

// LDS byte address of a shared-memory pointer, and loads from such an address (a
// constant added to one base register becomes the instruction's offset field).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS uint8_t*)p;
}
__device__ __forceinline__ v4i lds_ld16(uint32_t a) {
  return *(const LDS_AS v4i*)(uintptr_t)a;
}
__device__ __forceinline__ v4s lds_tr16(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS v4s*)(uintptr_t)a);
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
// wait states after a VALU write of an SGPR the load reads; nt marks the read-once
// stream of cache pages non-temporal.
__device__ __forceinline__ void dma16(uint64_t sbase, uint32_t voff, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
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

// (IEEE maximum: one v_maximum3_f32, where fmaxf would first quiet both swapped values)
__device__ __forceinline__ float group_max4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
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

struct BWItem {
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

// ------------------------------------------------------------------ QK waves
template <int NT>
__device__ __forceinline__ void bw_qk(const BWItem& it, BWSmem<NT>& sm) {
  constexpr int kQKT = BWRoles<NT>::kQKT;
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
  // rot(16 + l16) = rot(l16). Latent steps (kk < 16) never wrap.
  const int rot = rot_of(l16);
  const uint32_t pages0 = lds_addr(sm.pages[0]);
  const uint32_t k_lat = pages0 + l16 * kRowB + 16 * (g + rot);
  uint32_t k_rope[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    k_rope[r] = pages0 + l16 * kRowB + 16 * ((64 + 4 * r + g + rot) % kChunks);

  int stage_off = 0;  // byte offset of step st's stage; advanced per step
  const v2bf ones = {(__bf16)1.f, (__bf16)1.f};
  // One step. Token tile 0's MFMAs run first; the first half of its softmax (scores,
  // tile maximum c, x = 2^(t - c + 8)) runs between token tile 1's MFMAs. kMasked: the
  // page holds keys some row may not see (split end, causal limit).
  auto qk_step = [&](int st, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const int tok_page = (p_first + st) * kPage;
    v4f acc[kQKT][2];
#pragma unroll
    for (int k = 0; k < kQKT; ++k) acc[k][0] = acc[k][1] = v4f{0.f, 0.f, 0.f, 0.f};
    float t[kQKT][2][4], x[kQKT][2][4], c[kQKT][2], xsum[kQKT][2];
    // K fragments of token row 16 tt + l16, two steps of the dot product ahead
    v4i kf[3];
    auto kload = [&](int tt, int kk, v4i& f) {
      f = lds_ld16((kk < 16 ? k_lat + 64 * kk : k_rope[kk - 16]) + stage_off + 16 * tt * kRowB);
    };
    auto mfma_kk = [&](int tt, int kk) {
#pragma unroll
      for (int k = 0; k < kQKT; ++k)
        acc[k][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf8(kf[kk % 3]), as_bf8(qf[k][kk]), acc[k][tt], 0, 0, 0);
    };
    // softmax, first half, of (tile k, token tile tt) in four slices
    auto part1 = [&](int k, int tt, int slice) {
      if (slice == 0) {
        const int tok0 = tok_page + 16 * tt + 4 * g;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float v = acc[k][tt][jj] * it.scale_log2;
          if (kMasked && (tok0 + jj >= lim_q[k] || tok0 + jj < it.t0)) v = -INFINITY;
          t[k][tt][jj] = v;
        }
        c[k][tt] = __builtin_elementwise_maximum(  // IEEE maximum: no quieting
            __builtin_elementwise_maximum(t[k][tt][0], t[k][tt][1]),
            __builtin_elementwise_maximum(t[k][tt][2], t[k][tt][3]));
      } else if (slice == 1) {
        c[k][tt] = ceilf(group_max4(c[k][tt]));  // -inf when no key of the tile is visible
      } else if (slice == 2) {
        const float off = 8.f - (c[k][tt] == -INFINITY ? 0.f : c[k][tt]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) x[k][tt][jj] = t[k][tt][jj] + off;
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) x[k][tt][jj] = __builtin_amdgcn_exp2f(x[k][tt][jj]);  // exp2(-inf) = 0
        xsum[k][tt] = (x[k][tt][0] + x[k][tt][1]) + (x[k][tt][2] + x[k][tt][3]);
      }
    };
    // token tile 0
    kload(0, 0, kf[0]);
    kload(0, 1, kf[1]);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      if (kk + 2 < kKSteps) kload(0, kk + 2, kf[(kk + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_kk(0, kk);
      __builtin_amdgcn_sched_barrier(0);
    }
    // token tile 1, with slices of token tile 0's softmax from dot-product step 2 on
    kload(1, 0, kf[0]);
    kload(1, 1, kf[1]);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      if (kk + 2 < kKSteps) kload(1, kk + 2, kf[(kk + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
      mfma_kk(1, kk);
      const int sl = kk - 2;
      if (sl >= 0 && sl < 4 * kQKT) part1(sl / 4, 0, sl % 4);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int k = 0; k < kQKT; ++k) part1(k, 1, sl);
    // second half: the new running maximum m, P~ = BF16(x 2^(c - m)), sums, rescale
#pragma unroll
    for (int k = 0; k < kQKT; ++k) {
      const float mn = fmaxf(m_run[k], fmaxf(c[k][0], c[k][1]));
      const float al = mn == m_run[k] ? 1.f : pow2_diff(m_run[k], mn);  // 1: O unchanged
      const int row = (qw * kQKT + k) * kTileRows + l16;
      float xs = 0.f, ps = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float sc = pow2_diff(c[k][tt], mn);  // 2^(c - m), exact
        const v2bf p0 = __builtin_convertvector((v2f){x[k][tt][0] * sc, x[k][tt][1] * sc}, v2bf);
        const v2bf p1 = __builtin_convertvector((v2f){x[k][tt][2] * sc, x[k][tt][3] * sc}, v2bf);
        ps = __builtin_amdgcn_fdot2_f32_bf16(p0, ones, ps, false);
        ps = __builtin_amdgcn_fdot2_f32_bf16(p1, ones, ps, false);
        xs += xsum[k][tt] * sc;
        *(uint2*)(sm.ptile[st & 1] + row * kPRowB + 16 * g + 8 * tt) =
            make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
      }
      xs = group_sum4(xs);
      ps = group_sum4(ps);
      if (g == 0) sm.alpha[st & 1][row] = al;
      l_run[k] = l_run[k] * al + xs;
      lt_run[k] = lt_run[k] * al + ps;
      m_run[k] = mn;
    }
    stage_off = stage_off == (kStages - 1) * kPageB ? 0 : stage_off + kPageB;
  };
  auto qk = [&](int st) {
    const int tok_page = (p_first + st) * kPage;
    if (tok_page + kPage > lim_all || tok_page < it.t0) qk_step(st, std::true_type{});
    else qk_step(st, std::false_type{});
  };

  __builtin_amdgcn_s_setprio(2);  // the QK waves pace the step: issue first on their SIMD
  block_sync_lds();               // step 0 landed
  if (nsteps > 0) qk(0);
  for (int st = 0; st < nsteps; ++st) {
    block_sync_lds();
    if (st + 1 < nsteps) qk(st + 1);
  }

  // (m, l, l~) of rows 2 qw 16 + 16 k + l16; m is the maximum O is scaled to
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
  constexpr int kDT = 16;       // 16-dim tiles per PV wave
  constexpr int kDMA = R::kDMA;
  const PlanDev& P = *it.P;
  const int g = it.g, l16 = it.l16, lane = it.lane;
  const int nsteps = it.nsteps, p_first = it.p_first, p_end = it.p_end, t1 = it.t1;
  const int pv = it.w - R::kQKW;
  const int rt0 = (pv >> 1) * kRT;  // group pv >> 1
  const int dh = pv & 1;

  // Direct-to-LDS loads k = pv kDMA + i of a step: LDS bytes [1024 k, 1024 k + 1024) of
  // the stage; lane i fills 16-byte slot s = 64 k + i, which holds chunk
  // (s % 72 - rot(s / 72)) mod 72 of token row s / 72.
  uint32_t doff[kDMA];
#pragma unroll
  for (int i = 0; i < kDMA; ++i) {
    const int slot = (pv * kDMA + i) * 64 + lane;
    const int n = slot / kChunks, pos = slot - n * kChunks;
    int c = pos - rot_of(n);
    if (c < 0) c += kChunks;
    doff[i] = (uint32_t)(n * kRowB + 16 * c);
  }
  const uint32_t pages0 = lds_addr(sm.pages[0]);
  auto issue_one = [&](uint64_t gp, uint32_t stage_base, int i) {
    dma16(gp, doff[i], stage_base + (uint32_t)((pv * kDMA + i) * 1024));
  };
  auto page_id = [&](int st) -> int64_t { return it.btb[min(p_first + st, p_end - 1)]; };
  auto stage_of = [&](int st) -> uint32_t { return pages0 + (uint32_t)((st % kStages) * kPageB); };
  // rows past the split's end (the tail of its last page) read as zero V
  auto zero_tail = [&](int st) {
    const int valid = t1 - (p_first + st) * kPage;
    if (valid >= kPage) return;
    uint8_t* stage = sm.pages[st % kStages];
    for (int off = valid * kRowB + 16 * (pv * 64 + lane); off < kPageB; off += 16 * 64 * R::kPVW)
      *(v4i*)(stage + off) = v4i{0, 0, 0, 0};
  };
  // rows of the first page before a key window's start read as zero V as well
  auto zero_head = [&]() {
    const int skip = it.t0 - p_first * kPage;
    uint8_t* stage = sm.pages[0];
    for (int off = 16 * (pv * 64 + lane); off < skip * kRowB; off += 16 * 64 * R::kPVW)
      *(v4i*)(stage + off) = v4i{0, 0, 0, 0};
  };

  v4f acc[kRT][kDT];
#pragma unroll
  for (int k = 0; k < kRT; ++k)
#pragma unroll
    for (int d = 0; d < kDT; ++d) acc[k][d] = v4f{0.f, 0.f, 0.f, 0.f};
  // transposed V reads: lane (16 G + u), read r addresses token 16 r + 4 G + u / 4 and
  // dims 16 D + 4 (u % 4) .. + 3 (chunk 2 D + (u % 4) / 2, rotated, never wrapping);
  // lane 16 G + u receives dim 16 D + u of tokens 16 r + 4 G .. 16 r + 4 G + 3
  uint32_t tr_base[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 16 * r + 4 * g + (l16 >> 2);
    tr_base[r] = (uint32_t)(t * kRowB + 16 * (((l16 & 3) >> 1) + rot_of(t)) + 8 * (l16 & 1) +
                            512 * dh);
  }

  // one step: rescale O where a row's maximum moved, O += P~ V over the stage's page,
  // with the direct-to-LDS loads of step st + 3 (when dma) issued between the MFMAs
  auto pv_step = [&](int st, bool dma, uint64_t gp) {
    const int pb = st & 1;
    v8bf pa[kRT];
#pragma unroll
    for (int k = 0; k < kRT; ++k) {
      const int rt = rt0 + k;
      const float4 al = *(const float4*)&sm.alpha[pb][rt * kTileRows + 4 * g];
      if (__builtin_amdgcn_ballot_w64(al.x != 1.f || al.y != 1.f || al.z != 1.f || al.w != 1.f) != 0) {
#pragma unroll
        for (int d = 0; d < kDT; ++d) {
          acc[k][d][0] *= al.x; acc[k][d][1] *= al.y;
          acc[k][d][2] *= al.z; acc[k][d][3] *= al.w;
        }
      }
      pa[k] = as_bf8(ld16(sm.ptile[pb], (rt * kTileRows + l16) * kPRowB + 16 * g));
    }
    const uint32_t sb = stage_of(st);
    const uint32_t dst = stage_of(st + 3);
    const uint32_t v0 = sb + tr_base[0], v1 = sb + tr_base[1];
    v4s vr[3][2];
    auto vload = [&](int d, v4s (&f)[2]) {
      f[0] = lds_tr16(v0 + 32 * d);
      f[1] = lds_tr16(v1 + 32 * d);
    };
    vload(0, vr[0]);
    vload(1, vr[1]);
#pragma unroll
    for (int d = 0; d < kDT; ++d) {
      if (d + 2 < kDT) vload(d + 2, vr[(d + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
      const v2u x0 = __builtin_bit_cast(v2u, vr[d % 3][0]);
      const v2u x1 = __builtin_bit_cast(v2u, vr[d % 3][1]);
      const v4i vb = v4i{(int)x0.x, (int)x0.y, (int)x1.x, (int)x1.y};
#pragma unroll
      for (int k = 0; k < kRT; ++k)
        acc[k][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[k], as_bf8(vb), acc[k][d], 0, 0, 0);
      if (d < kDMA && dma) issue_one(gp, dst, d);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: 1 + nsteps barriers, like the QK waves; a step's page id is read one
  // step before its loads are issued
  int64_t nid = 0;
#pragma unroll
  for (int pre = 0; pre < kStages - 1; ++pre) {
    if (pre < nsteps) {
      const uint64_t gp = uniform_addr(it.kv + page_id(pre) * kPageB);
#pragma unroll
      for (int i = 0; i < kDMA; ++i) issue_one(gp, stage_of(pre), i);
    }
  }
  if (nsteps > kStages - 1) nid = page_id(kStages - 1);
  // step 0 landed: the loads of steps 1 and 2 may still be in flight
  if (nsteps > 2) wait_vmcnt<2 * kDMA>();
  else if (nsteps > 1) wait_vmcnt<kDMA>();
  else wait_vmcnt<0>();
  block_sync_lds();
  if (nsteps == 1) zero_tail(0);
  if (nsteps > 0) zero_head();
  for (int st = 0; st < nsteps; ++st) {
    // step st + 1 landed; step st + 2's loads may stay in flight
    if (st + 2 < nsteps) wait_vmcnt<kDMA>(); else wait_vmcnt<0>();
    block_sync_lds();
    if (st + 2 == nsteps) zero_tail(st + 1);
    const bool dma = st + 3 < nsteps;
    const uint64_t gp = uniform_addr(it.kv + nid * kPageB);
    if (dma && st + 4 < nsteps) nid = page_id(st + 4);
    pv_step(st, dma, gp);
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
                         const int32_t* __restrict__ q_lens,
                         const int32_t* __restrict__ kv_bounds, float scale_log2_arg,
                         float* __restrict__ ws_o, float* __restrict__ ws_stats) {
  __shared__ BWSmem<NT> sm;
  const PlanDev& P = kDev ? *pdev : Parg;
  const float scale_log2 = kDev ? *scale_dev * 1.4426950408889634f : scale_log2_arg;
  BWItem it;
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

  if (it.w < BWRoles<NT>::kQKW) bw_qk<NT>(it, sm);
  else bw_pv<NT>(it, sm);
}

}  // namespace

int launch_partial_bf16_wide(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                             const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                             float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                             const DeviceArgs* dev, const int32_t* q_lens,
                        const int32_t* kv_bounds) {
  const PlanDev& P = plan.dev;
  const int slots = (P.total_parts * P.subs + 7) / 8;
  const dim3 grid(8 * slots * P.tiles);
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const PlanDev* pd = dev ? dev->plan : nullptr;
  const float* sd = dev ? dev->softmax_scale : nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (P.nt == 4) {
    const dim3 block(BWRoles<4>::kThreads);
    if (dev)
      hipLaunchKernelGGL((partial_bf16_wide_kernel<4, true>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
    else
      hipLaunchKernelGGL((partial_bf16_wide_kernel<4, false>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
  } else {
    const dim3 block(BWRoles<6>::kThreads);
    if (dev)
      hipLaunchKernelGGL((partial_bf16_wide_kernel<6, true>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
    else
      hipLaunchKernelGGL((partial_bf16_wide_kernel<6, false>), grid, block, 0, st, P, pd, sd, q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
