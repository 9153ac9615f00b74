// Split-KV partial kernel for MLA decode, wide row blocks (64 or 96 query rows), gfx950.
//
// Computes what the narrow kernel (partial.hip) computes, per (request b, split s,
// block of 16 NT query rows): the online-softmax state of TensorRT-LLM PR #20380
// "trtllm-gen FMHA: split the KV partials of a row across thread groups in
// fmhaReductionKernel" (Description: per-row max, sum and unnormalised O) over the
// split's keys, with the causal limit of the MTP verify shape (issue #20510 "CuTe DSL
// FP8 MLA decode slower after #19338", Setup). P~ is the two-term E4M3 form of the FP16
// rounding of x = 2^(t - c + 8) (the QK waves hand x to the PV waves as FP16); it
// depends only on the page's own scores, so the partials are the same under every
// split plan.
//
// Why a second kernel: with q = 8 (and with 96 heads) a request has 96-768 rows. The
// narrow kernel stages the KV through LDS once per 32 rows; here one staged page
// feeds 64 or 96 rows, so each KV byte crosses HBM->L2->LDS once per 96 rows and the
// MFMA units, not the gather, set the pace (these shapes need ~300 flop per KV byte).
//
// Design for gfx950: one workgroup of 2 + NT wavefronts (at most 2 per SIMD) per item.
//  * Gather: direct-to-LDS loads (global_load_lds_dwordx4, 1 KB of one page per
//    instruction) into a 3-stage ring of 2-page steps, issued by the PV waves two steps
//    ahead. Rows stay 576 bytes (the load writes LDS contiguously); instead, 16-byte
//    chunk c of token row n sits at chunk (c + ((n >> 2) & 3)) mod 36, which puts the
//    16 rows of an operand read, and the 16 consecutive rows of a transposed V read, on
//    distinct LDS banks. VGPR staging would need ~290 VGPRs per step that the MFMA
//    waves use for operands and accumulators.
//  * QK^T: QK wave q owns row tiles [q NT/2, (q + 1) NT/2) (Q^T of all in VGPRs) and
//    computes S^T = K Q^T for both pages of the step: the 512 latent bytes on
//    v_mfma_scale_f32_16x16x128_f8f6f4, the 64 rope bytes on two
//    v_mfma_f32_16x16x32_fp8_fp8; every K fragment read from LDS feeds NT/2 MFMAs. Softmax as in the narrow kernel:
//    per (row, page) c = ceil(max t), x = 2^(t - c + 8), written to LDS as FP16; the
//    PV waves split it into P~ = hi + lo / 16 (hi = e4m3(x), lo = e4m3(16 (x - hi)))
//    with the packed FP16 conversions of gfx950 (x - hi is exact in FP16), which keeps
//    the quantisation work off the QK waves.
//    The QK waves also keep each row's running maximum m (an integer) and l = sum x,
//    and publish per step the rescale factor 2^(m_old - m_new) and the page exponents
//    c_page - m_new; l~ = sum P~ comes from one PV MFMA against a tile of ones.
//  * PV: NT waves; wave (pair pp, half dh) accumulates O for row tiles 2 pp, 2 pp + 1
//    and dims [256 dh, 256 dh + 256): every transposed V read feeds two MFMAs. The page
//    exponents enter through the E8M0 block scales.
//  * Token order inside an MFMA K block: position 16 G + j of a step (G = lane group)
//    holds token 32 (G >> 1) + 16 (j >> 3) + 8 (G & 1) + (j & 7), so the 32 lanes that
//    one transposed read serves at a time read 16 consecutive token rows.
//  * Skewed single-barrier pipeline: iteration s runs QK/softmax of step s + 1 and PV of
//    step s; P~ and the page maxima are double-buffered.
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
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kStepPages = 2;
constexpr int kStepBytes = kStepPages * kPageBytes;  // 36864
constexpr int kStages = 3;
constexpr int kChunks = kDQK / 16;                   // 36 chunks of 16 bytes per row
constexpr int kStepLoads = kStepBytes / 1024;        // 36 wave-wide 16-byte loads per step
constexpr int kPageLoads = kPageBytes / 1024;        // 18 of them per page
static_assert(kStepLoads * 1024 == kStepBytes && kPageBytes % 1024 == 0, "1 KB loads tile a step");
constexpr int kPRow = 144;                           // row of x: 64 FP16 + 16 bytes of pad
constexpr int kOnesE4M3 = 0x38383838;                // four E4M3 1.0

// Roles (at most 2 waves per SIMD, so every wave may hold 256 VGPRs):
//  * 2 QK waves; wave q holds Q^T of row tiles [q NT/2, (q + 1) NT/2) in registers.
//  * NT PV waves; wave (pair pp, half dh) accumulates O of row tiles 2 pp, 2 pp + 1 and
//    dims [256 dh, 256 dh + 256), keeps l~ of row tile 2 pp + dh, and issues 36 / NT of
//    the step's direct-to-LDS loads.
template <int NT>
struct WRoles {
  static_assert(NT == 4 || NT == 6, "wide row blocks hold 4 or 6 row tiles");
  static constexpr int kQKW = 2;                      // QK waves
  static constexpr int kQKT = NT / 2;                 // row tiles per QK wave
  static constexpr int kPVW = NT;                     // PV waves
  static constexpr int kWaves = kQKW + kPVW;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kDMA = kStepLoads / kPVW;      // 1 KB loads per PV wave per step
  static_assert(kDMA * kPVW == kStepLoads && kPageLoads % kDMA == 0, "a wave's loads stay in one page");
  static_assert(kWaves <= 8, "two waves per SIMD");
};

template <int NT>
struct __attribute__((aligned(16))) WSmem {
  uint8_t pages[kStages][kStepBytes];
  uint8_t ptile[2][NT * kTileRows * kPRow];
  float alpha[2][NT * kTileRows];              // per row: 2^(m_old - m_new) of the step
  float2 sc[2][NT * kTileRows];                // per row: c_page - m_new of both pages
};

__device__ __forceinline__ int rot_of(int n) { return (n >> 2) & 3; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier ordering LDS traffic only (the direct-to-LDS loads still in flight
// for later stages are awaited explicitly by the waves that issued them).
__device__ __forceinline__ void block_sync_lds() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wave-wide direct-to-LDS load: lane i's 16 bytes at sbase + voff land at LDS
// byte address lds_base + 16 i. Issued from inline asm so that the compiler's
// wait-count pass does not drain it at every LDS access; M0 carries the LDS base and is
// restored. The s_nop covers the wait states a vector memory instruction needs after a
// VALU write of an SGPR it reads (the base may come from v_readfirstlane), which the
// compiler does not insert in front of inline assembly. The nt (non-temporal) policy
// marks the stream of cache pages as read-once, as the narrow kernels' loads are
// (measured: 1-2% faster on the q = 8 shapes, bit-identical).
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

// A wave-uniform 64-bit address in SGPRs (both halves zero-extended).
__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

__device__ __forceinline__ v4i ld16(const uint8_t* base, int off) {
  return *(const v4i*)(base + off);
}

// LDS byte address of a shared-memory pointer, and a transposed read from such an
// address (a constant added to one base register becomes the instruction's offset).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS uint8_t*)p;
}
__device__ __forceinline__ v2i lds_tr8(uint32_t a) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(uintptr_t)a);
}

__device__ __forceinline__ v8i cat8(v4i a, v4i b) {
  return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

// Max / sum over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48) with the
// VALU lane swaps of gfx950 instead of LDS permutes.
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

struct WItem {
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

// ------------------------------------------------------------------ QK waves
// QK wave qw: S^T = K Q^T of both pages of a step for row tiles qw NT/2 + k, the
// per-page softmax (P~ to LDS), and the row bookkeeping: running max m (integer) and l,
// with the step's rescale factor 2^(m_old - m_new) and the block-scale exponents
// c_page - m_new published for the PV waves. Writes the rows' (m, l) at the end.
template <int NT>
__device__ __forceinline__ void wide_qk(const WItem& it, WSmem<NT>& sm) {
  using R = WRoles<NT>;
  const PlanDev& P = *it.P;
  const int g = it.g, l16 = it.l16, qw = it.w;
  const int nsteps = it.nsteps, p_first = it.p_first, t1 = it.t1;

  // Q^T fragments of row tiles qw NT/2 + k: lane (row l16, group g) holds bytes
  // [32 g, 32 g + 32) of each 128-byte K step of its row (latent, 4 scaled FP8 MFMAs of
  // K = 128) and 8 bytes of each half of the rope (2 FP8 MFMAs of K = 32).
  constexpr int kT = R::kQKT;
  v8i qf[kT][4];
  long qr[kT][2];
  int lim_q[kT];
#pragma unroll
  for (int k = 0; k < kT; ++k) {
    const int qrow = it.row0 + (qw * kT + k) * kTileRows + l16;
    const bool valid = qrow < P.rows;
    const uint8_t* qp = it.q + ((int64_t)it.b * P.rows + (valid ? qrow : 0)) * kDQK;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      v4i a = ld16(qp, 128 * c4 + 32 * g);
      v4i c = ld16(qp, 128 * c4 + 32 * g + 16);
      if (!valid) { a = 0; c = 0; }
      qf[k][c4] = cat8(a, c);
    }
    // rope: two K = 32 steps, lane group g holds bytes [8 g, 8 g + 8) of each half
    qr[k][0] = valid ? *(const long*)(qp + 512 + 8 * g) : 0;
    qr[k][1] = valid ? *(const long*)(qp + 544 + 8 * g) : 0;
    // causal limit of the row: query j of a request with qb queries sees tokens
    // < L - qb + j + 1; rows past the request's queries see none
    const int jq = valid ? qrow / P.heads : 0;
    lim_q[k] = jq < it.qb ? min(t1, it.L - it.qb + jq + 1) : kNoKey;
  }
  // below this token no row of the wave needs a mask
  const int first_row = min(it.row0 + qw * kT * kTileRows, P.rows - 1);
  const int last_row = min(it.row0 + (qw + 1) * kT * kTileRows, P.rows) - 1;
  const int lim_all = last_row / P.heads >= it.qb
      ? kNoKey : min(t1, it.L - it.qb + first_row / P.heads + 1);

  // K operand offsets inside a token row (swizzled chunks; rot depends on l16 only).
  const int rot = l16 >> 2;
  const int k_off = 16 * (2 * g + rot);  // + 128 c4 (+ 16): no wrap for c4 < 4
  const int r_off0 = 16 * ((32 + (g >> 1) + rot) % kChunks) + 8 * (g & 1);
  const int r_off1 = 16 * ((34 + (g >> 1) + rot) % kChunks) + 8 * (g & 1);

  // row bookkeeping of rows (qw NT/2 + k) 16 + l16: m identical in the four lane groups,
  // l kept per lane over the lane's own tokens and summed over the groups at the end
  float m_run[kT], l_run[kT];
#pragma unroll
  for (int k = 0; k < kT; ++k) { m_run[k] = -INFINITY; l_run[k] = 0.f; }

  auto qk_step = [&](int st) {
    const uint8_t* stage = sm.pages[st % kStages];
    float cpg[kT][kStepPages], xs[kT][kStepPages];
    // K fragments of block (page p, token tile tt): 4 x 32 latent bytes + 2 x 8 rope
    // bytes per lane. The fragments of the next block are read while this block's MFMAs
    // run (two buffers), so the LDS latency is paid once per step, not once per block.
    struct KFrag { v8i kf[4]; long r0, r1; };
    auto load_frag = [&](int p, int tt, KFrag& f) {
      const uint8_t* rowp = stage + p * kPageBytes + (16 * tt + l16) * kDQK;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        f.kf[c4] = cat8(ld16(rowp, k_off + 128 * c4), ld16(rowp, k_off + 128 * c4 + 16));
      f.r0 = *(const long*)(rowp + r_off0);
      f.r1 = *(const long*)(rowp + r_off1);
    };
    // QK^T of block (page p, token tile tt) into out[k] for the wave's row tiles
    auto mfma_block = [&](const KFrag& f, v4f (&out)[kT]) {
      v4f a4[kT];
#pragma unroll
      for (int k = 0; k < kT; ++k) a4[k] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
        for (int k = 0; k < kT; ++k)
          a4[k] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.kf[c4], qf[k][c4], a4[k], 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int k = 0; k < kT; ++k) {
        const v4f a = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(f.r0, qr[k][0], a4[k], 0, 0, 0);
        out[k] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(f.r1, qr[k][1], a, 0, 0, 0);
      }
    };
    // softmax of page p from its two token tiles: P~ to LDS, (c, sum x) kept
    auto softmax_page = [&](int p, const v4f (&s0)[kT], const v4f (&s1)[kT]) {
      // lane holds S[row l16][page token 16 tt + 4 g + jj]
      const int tok_page = (p_first + st * kStepPages + p) * kPage;
      const bool need_mask = tok_page + kPage > lim_all || tok_page < it.t0;
#pragma unroll
      for (int k = 0; k < kT; ++k) {
        float t[2][4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          t[0][jj] = s0[k][jj] * it.scale_log2;
          t[1][jj] = s1[k][jj] * it.scale_log2;
        }
        if (need_mask) {  // uniform: only pages that reach the split's end or a causal limit
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              if (tok_page + 16 * tt + 4 * g + jj >= lim_q[k] ||
                  tok_page + 16 * tt + 4 * g + jj < it.t0)
                t[tt][jj] = -INFINITY;
        }
        // IEEE maximum: no quieting of the values that come through the mask branch
        float mx = __builtin_elementwise_maximum(
            __builtin_elementwise_maximum(__builtin_elementwise_maximum(t[0][0], t[0][1]),
                                          __builtin_elementwise_maximum(t[0][2], t[0][3])),
            __builtin_elementwise_maximum(__builtin_elementwise_maximum(t[1][0], t[1][1]),
                                          __builtin_elementwise_maximum(t[1][2], t[1][3])));
        mx = group_max4(mx);
        const float c = ceilf(mx);  // -inf when no key of the page is visible to the row
        const float off = 8.f - (c == -INFINITY ? 0.f : c);
        float sx = 0.f;
        const int row = (qw * kT + k) * kTileRows + l16;
        // page token 16 tt + 4 g + jj goes to K position 32 p + 16 (g >> 1) + 8 tt + 4 (g & 1) + jj;
        // the QK wave hands x over as FP16 (2 bytes per position), the PV waves split it
        uint8_t* prow = sm.ptile[st & 1] + row * kPRow + 2 * (32 * p + 16 * (g >> 1) + 4 * (g & 1));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float x[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            x[jj] = __builtin_amdgcn_exp2f(t[tt][jj] + off);  // v_exp_f32; exp2(-inf) = 0
            sx += x[jj];
          }
          *(v2h*)(prow + 16 * tt) = v2h{(_Float16)x[0], (_Float16)x[1]};
          *(v2h*)(prow + 16 * tt + 4) = v2h{(_Float16)x[2], (_Float16)x[3]};
        }
        cpg[k][p] = c;
        xs[k][p] = sx;
      }
    };
    // blocks 0 .. 3 = (page 0, tt 0), (0, 1), (1, 0), (1, 1). The K reads of blocks 1
    // and 2 go out before the previous block's MFMAs; page 0's softmax (VALU) is issued
    // with block 2's MFMAs so that it runs while the matrix cores work on page 1; block
    // 3's reads follow it (holding them earlier would not fit the register budget).
    KFrag fa, fb;
    v4f s00[kT], s01[kT], s10[kT], s11[kT];
    load_frag(0, 0, fa);
    load_frag(0, 1, fb);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(fa, s00);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(1, 0, fa);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(fb, s01);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(fa, s10);
    softmax_page(0, s00, s01);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(1, 1, fb);
    __builtin_amdgcn_sched_barrier(0);
    mfma_block(fb, s11);
    softmax_page(1, s10, s11);
    // step bookkeeping: new running max, rescale factor, page exponents, l
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const float mn = fmaxf(m_run[k], fmaxf(cpg[k][0], cpg[k][1]));
      const float al = mn == m_run[k] ? 1.f : pow2_diff(m_run[k], mn);
      const float w0 = pow2_diff(cpg[k][0], mn), w1 = pow2_diff(cpg[k][1], mn);
      l_run[k] = l_run[k] * al + xs[k][0] * w0 + xs[k][1] * w1;
      m_run[k] = mn;
      const int row = (qw * kT + k) * kTileRows + l16;
      if (g == 0) {
        sm.alpha[st & 1][row] = al;
        sm.sc[st & 1][row] = make_float2(cpg[k][0] == -INFINITY ? -INFINITY : cpg[k][0] - mn,
                                         cpg[k][1] == -INFINITY ? -INFINITY : cpg[k][1] - mn);
      }
    }
  };

  // ---- pipeline: 1 + nsteps barriers, like the PV waves
  __builtin_amdgcn_s_setprio(2);  // the QK waves pace the step: issue first on their SIMD
  block_sync_lds();  // step 0 landed
  if (nsteps > 0) qk_step(0);
  for (int st = 0; st < nsteps; ++st) {
    block_sync_lds();
    if (st + 1 < nsteps) qk_step(st + 1);
  }

  // ---- (m, l) of the wave's rows (l~ comes from the PV waves)
#pragma unroll
  for (int k = 0; k < kT; ++k) l_run[k] = group_sum4(l_run[k]);
  if (g == 0) {
    const int64_t part_row0 = (int64_t)it.part * P.rows;
#pragma unroll
    for (int k = 0; k < kT; ++k) {
      const int row = it.row0 + (qw * kT + k) * kTileRows + l16;
      if (row < P.rows)
        *(float2*)(it.ws_stats + (part_row0 + row) * kStatStride) = make_float2(m_run[k], l_run[k]);
    }
  }
}

// ------------------------------------------------------------------ PV waves
// PV wave (pair pv >> 1, half pv & 1): O of row tiles rt0, rt0 + 1 and dims
// [256 dh, 256 dh + 256), rescaled by the QK waves' per-step factors; l~ of row tile
// rt0 + dh; and loads pv kDMA .. pv kDMA + kDMA - 1 of every step.
template <int NT>
__device__ __forceinline__ void wide_pv(const WItem& it, WSmem<NT>& sm) {
  using R = WRoles<NT>;
  constexpr int kRT = 2;   // row tiles per PV wave
  constexpr int kDT = 16;  // 16-dim tiles per PV wave
  const PlanDev& P = *it.P;
  const int g = it.g, l16 = it.l16;
  const int nsteps = it.nsteps, p_first = it.p_first, t1 = it.t1;
  const int pv = it.w - R::kQKW;
  const int rt0 = (pv >> 1) * kRT;  // row tiles [rt0, rt0 + 2)
  const int dh = pv & 1;             // dims [256 dh, 256 dh + 256)
  const int lane = it.lane, p_end = it.p_end;

  // Direct-to-LDS loads: loads k = pv kDMA + i of every step, all in page (pv kDMA) / 18;
  // load k fills LDS bytes [1024 k, 1024 k + 1024) of the stage. Source offsets inside
  // the page, 16 bits each, two per register.
  uint32_t src2[(R::kDMA + 1) / 2];
#pragma unroll
  for (int i = 0; i < R::kDMA; i += 2) {
    uint32_t v = 0;
#pragma unroll
    for (int h = 0; h < 2 && i + h < R::kDMA; ++h) {
      const int k = pv * R::kDMA + i + h;
      const int slot = (k % kPageLoads) * 64 + lane;  // 16-byte slot of the page in LDS
      const int n = slot / kChunks, pos = slot % kChunks;
      int c = pos - rot_of(n);
      if (c < 0) c += kChunks;
      v |= (uint32_t)(n * kDQK + 16 * c) << (16 * h);
    }
    src2[i / 2] = v;
  }
  const bool ld_page_b = (pv * R::kDMA) >= kPageLoads;
  // block-table index of this wave's page in step st (odd tail: reload page a)
  auto page_of = [&](int st) {
    const int pa = p_first + st * kStepPages;
    return ld_page_b ? min(pa + 1, p_end - 1) : pa;
  };
  const uint32_t pages0 = lds_addr(sm.pages[0]);
  auto stage_of = [&](int st) -> uint32_t { return pages0 + (uint32_t)((st % kStages) * kStepBytes); };
  auto issue_one = [&](uint64_t gp, uint32_t stage_base, int i) {
    const uint32_t off = (src2[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
    dma16(gp, off, stage_base + (uint32_t)((pv * R::kDMA + i) * 1024));
  };
  auto issue = [&](int st, int64_t id) {
    const uint64_t gp = uniform_addr(it.kv + id * kPageBytes);
#pragma unroll
    for (int i = 0; i < R::kDMA; ++i) issue_one(gp, stage_of(st), i);
  };
  // token rows of a step past the split's end (its last step) read as zero V: the
  // stage holds the step's 64 token rows back to back
  auto zero_tail = [&](int st) {
    const int valid = t1 - (p_first + st * kStepPages) * kPage;
    if (valid >= kStepPages * kPage) return;
    uint8_t* stage = sm.pages[st % kStages];
    for (int off = valid * kDQK + 16 * (pv * 64 + lane); off < kStepBytes; off += 16 * 64 * R::kPVW)
      *(v4i*)(stage + off) = v4i{0, 0, 0, 0};
  };
  // so do the rows of the first page before a key window's start
  auto zero_head = [&]() {
    const int skip = it.t0 - p_first * kPage;
    uint8_t* stage = sm.pages[0];
    for (int off = 16 * (pv * 64 + lane); off < skip * kDQK; off += 16 * 64 * R::kPVW)
      *(v4i*)(stage + off) = v4i{0, 0, 0, 0};
  };

  v4f acc[kRT][kDT];
  v4f acc1 = v4f{0.f, 0.f, 0.f, 0.f};  // l~ of row tile rt0 + dh: ones product
#pragma unroll
  for (int k = 0; k < kRT; ++k)
#pragma unroll
    for (int d = 0; d < kDT; ++d) acc[k][d] = v4f{0.f, 0.f, 0.f, 0.f};
  // transposed V reads: lane (16 G + u), read r names token 16 r + 8 (G & 1) + u / 2 of
  // page G >> 1 and the 8-byte half u % 2 of a 16-dim chunk; it receives dim
  // 16 chunk + l16 for 8 tokens.
  int tr_base[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int t = 16 * r + 8 * (g & 1) + (l16 >> 1);
    tr_base[r] = (g >> 1) * kPageBytes + t * kDQK + 16 * (kDT * dh + rot_of(t)) + 8 * (l16 & 1);
  }

  // one step: O += P~ V over the stage's two pages, with the direct-to-LDS loads of
  // step st + 2 (when dma) issued together after the first dim tile's MFMAs
  auto pv_step = [&](int st, bool dma, uint64_t gp) {
    const int pb = st & 1;
    const uint32_t sb = stage_of(st), dst = stage_of(st + 2);
    const uint32_t v0 = sb + tr_base[0], v1 = sb + tr_base[1];
    // LDS reads of the step's small operands first (per row tile: the rescale factors of
    // result rows rt 16 + 4 g + jj, the page exponents of operand row rt 16 + l16 and
    // its 16 x values), then the first dim tiles' V, so that the P~ split's VALU work
    // covers the V reads' latency and no wait for the small reads also waits for V
    float4 al[kRT];
    float ep[kRT];  // page exponent of K block g = (term g >> 1, page g & 1)
    v4i xa[kRT], xb[kRT];
#pragma unroll
    for (int k = 0; k < kRT; ++k) {
      const int rt = rt0 + k;
      al[k] = *(const float4*)&sm.alpha[pb][rt * kTileRows + 4 * g];
      const float2 e = sm.sc[pb][rt * kTileRows + l16];
      const float ex = e.x, ey = e.y;
      ep[k] = (g & 1) ? ey : ex;
      const uint8_t* prow = sm.ptile[pb] + (rt * kTileRows + l16) * kPRow + 32 * g;
      xa[k] = ld16(prow, 0);
      xb[k] = ld16(prow, 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kPre = 2;
    v2i pre0[kPre], pre1[kPre];
#pragma unroll
    for (int d = 0; d < kPre; ++d) {
      pre0[d] = lds_tr8(v0 + 16 * d);
      pre1[d] = lds_tr8(v1 + 16 * d);
    }
    __builtin_amdgcn_sched_barrier(0);
    int sa[kRT];
    v8i pa[kRT];
#pragma unroll
    for (int k = 0; k < kRT; ++k) {
      // rescale when the running max moved
      const float4 a4 = al[k];
      const bool rescale = a4.x != 1.f || a4.y != 1.f || a4.z != 1.f || a4.w != 1.f;
      if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
        for (int d = 0; d < kDT; ++d) {
          acc[k][d][0] *= a4.x; acc[k][d][1] *= a4.y;
          acc[k][d][2] *= a4.z; acc[k][d][3] *= a4.w;
        }
        if (k == dh) {
          acc1[0] *= a4.x; acc1[1] *= a4.y; acc1[2] *= a4.z; acc1[3] *= a4.w;
        }
      }
      // E8M0 scale of K block g
      sa[k] = ep[k] == -INFINITY ? 127 : max(0, 127 + (int)ep[k] - 4 * (g >> 1));
      // P~ of K positions 16 g .. 16 g + 15 from the FP16 x the QK wave left:
      // hi = e4m3(x), lo = e4m3(16 (x - hi)); x - hi is exact in FP16, and the scaled
      // conversion divides by its scale (1/16 gives the factor 16)
      const int xw[8] = {xa[k].x, xa[k].y, xa[k].z, xa[k].w, xb[k].x, xb[k].y, xb[k].z, xb[k].w};
      int hw[4], lw[4];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const v2h x01 = __builtin_bit_cast(v2h, xw[2 * w4]);
        const v2h x23 = __builtin_bit_cast(v2h, xw[2 * w4 + 1]);
        v2s h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(v2s{0, 0}, x01, 1.0f, false);
        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(h, x23, 1.0f, true);
        const int hi = __builtin_bit_cast(int, h);
        const v2h d01 = x01 - __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
        const v2h d23 = x23 - __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
        v2s l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(v2s{0, 0}, d01, 0.0625f, false);
        l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(l, d23, 0.0625f, true);
        hw[w4] = hi;
        lw[w4] = __builtin_bit_cast(int, l);
      }
      pa[k] = v8i{hw[0], hw[1], hw[2], hw[3], lw[0], lw[1], lw[2], lw[3]};
      if (k == dh) {
        const v8i ones = v8i{kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3,
                             kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3};
        acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa[k], ones, acc1, 0, 0, 0, sa[k], 0, 127);
      }
    }
    // V: byte j of word w of the operand is step token 32 (g >> 1) + 16 (w >> 1) +
    // 8 (g & 1) + 4 (w & 1) + j; rows past the split's end were zeroed in LDS
#pragma unroll
    for (int d = 0; d < kDT; ++d) {
      const v2i b0 = d < kPre ? pre0[d < kPre ? d : 0] : lds_tr8(v0 + 16 * d);
      const v2i b1 = d < kPre ? pre1[d < kPre ? d : 0] : lds_tr8(v1 + 16 * d);
      const v8i vb = v8i{b0.x, b0.y, b1.x, b1.y, b0.x, b0.y, b1.x, b1.y};
#pragma unroll
      for (int k = 0; k < kRT; ++k)
        acc[k][d] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa[k], vb, acc[k][d], 0, 0, 0, sa[k], 0, 127);
      if (d == 0 && dma) {  // the step's loads go out together, after the first MFMAs
#pragma unroll
        for (int i = 0; i < R::kDMA; ++i) issue_one(gp, dst, i);
      }
    }
  };

  // ---- pipeline: 1 + nsteps barriers, like the QK waves. The page id of a step is
  // read one step before its loads are issued, so the issue never waits on it.
  int64_t nid = 0;
  if (nsteps > 0) issue(0, it.btb[page_of(0)]);
  if (nsteps > 1) issue(1, it.btb[page_of(1)]);
  if (nsteps > 2) nid = it.btb[page_of(2)];
  if (nsteps > 1) wait_vmcnt<R::kDMA>(); else wait_vmcnt<0>();  // step 0 landed
  block_sync_lds();
  if (nsteps == 1) zero_tail(0);
  if (nsteps > 0) zero_head();
  for (int st = 0; st < nsteps; ++st) {
    wait_vmcnt<0>();  // step st + 1 landed
    block_sync_lds();
    if (st + 2 == nsteps) zero_tail(st + 1);
    const bool dma = st + 2 < nsteps;
    const uint64_t gp = uniform_addr(it.kv + nid * kPageBytes);
    if (dma && st + 3 < nsteps) nid = it.btb[page_of(st + 3)];
    pv_step(st, dma, gp);
  }

  // ---- O partial rows rt 16 + 4 g + jj, dims 256 dh + 16 d + l16
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
        if (k == dh && l16 == 0) it.ws_stats[(part_row0 + row) * kStatStride + 2] = acc1[jj];
      }
    }
  }
}

// kDev: the plan and the softmax scale come from device memory (graph path).
template <int NT, bool kDev>
__global__ void __launch_bounds__(WRoles<NT>::kThreads, 1)
partial_wide_kernel(const PlanDev Parg, const PlanDev* __restrict__ pdev,
                    const float* __restrict__ scale_dev, const uint8_t* __restrict__ q,
                    const uint8_t* __restrict__ kv, const int32_t* __restrict__ bt,
                    int64_t bt_stride, const int32_t* __restrict__ kv_lens,
                    const int32_t* __restrict__ q_lens,
                    const int32_t* __restrict__ kv_bounds, float scale_log2_arg,
                    float* __restrict__ ws_o, float* __restrict__ ws_stats) {
  __shared__ WSmem<NT> sm;
  const PlanDev& P = kDev ? *pdev : Parg;
  const float scale_log2 = kDev ? *scale_dev * 1.4426950408889634f : scale_log2_arg;
  WItem it;
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

  if (it.w < WRoles<NT>::kQKW) wide_qk<NT>(it, sm);
  else wide_pv<NT>(it, sm);
}

}  // namespace

int launch_partial_wide(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                        const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                        float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                        const DeviceArgs* dev, const int32_t* q_lens,
                        const int32_t* kv_bounds) {
  const PlanDev& P = plan.dev;
  const int slots = (P.total_parts * P.subs + 7) / 8;  // graph plans: the capacity
  const dim3 grid(8 * slots * P.tiles);
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  const PlanDev* pd = dev ? dev->plan : nullptr;
  const float* sd = dev ? dev->softmax_scale : nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (P.nt == 4) {
    if (dev)
      hipLaunchKernelGGL((partial_wide_kernel<4, true>), grid, dim3(WRoles<4>::kThreads), 0, st, P, pd, sd,
                         q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
    else
      hipLaunchKernelGGL((partial_wide_kernel<4, false>), grid, dim3(WRoles<4>::kThreads), 0, st, P, pd, sd,
                         q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
  } else {
    if (dev)
      hipLaunchKernelGGL((partial_wide_kernel<6, true>), grid, dim3(WRoles<6>::kThreads), 0, st, P, pd, sd,
                         q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
    else
      hipLaunchKernelGGL((partial_wide_kernel<6, false>), grid, dim3(WRoles<6>::kThreads), 0, st, P, pd, sd,
                         q, kv, bt, bt_stride, kv_lens, q_lens, kv_bounds, scale_log2, ws_o, ws_stats);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
