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
// Design for gfx950: one workgroup of 8 wavefronts per work item, one work item per CU.
//  * Page gather: the split's pages stream through a 4-stage LDS ring of 2-page steps
//    (36 KB each) with 16-byte direct-to-LDS loads (global_load_lds_dwordx4); a page is
//    one contiguous 18 KB block of HBM, so every load is fully coalesced. Waves without
//    QK work issue the loads; block-table entries are read one step ahead. Within a
//    page, 16-byte chunk c of token row n sits at chunk (c + ((n >> 2) & 3)) mod 36 of
//    that row, which spreads the row-strided operand reads over the LDS banks.
//  * QK^T: QK wave (page p, row tile rt) forms the two 16-token tiles of S^T = K Q^T of
//    its page on v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3, fp32 accumulate), K straight
//    from LDS and Q^T resident in VGPRs; the 576-wide dot is 4 full MFMAs plus one whose
//    rope half is zero in both operands. Row tiles of the same work item share every
//    page staged in LDS, so KV is read from HBM once per 64 query rows.
//  * Softmax (exp2 domain, in-wave): per (row, page) c = ceil(max t over the page),
//    x = 2^(t - c + 8) in (0, 256], P~ = hi + lo/16 with hi = e4m3(x),
//    lo = e4m3(16 (x - hi)). P~ depends only on the page's own scores, so a token gets
//    bit-identical P~ under every split plan (splits hold whole pages). The row max is
//    kept on integers, m = max over pages of c, and the factor 2^(c - m) rides in the
//    MFMA's E8M0 block scale; all rescales are exact powers of two.
//  * PV: wavefront w owns output dims [64w, 64w + 64) for all rows of the work item.
//    One scaled MFMA covers 64 tokens of both terms: A bytes 0-15 hold hi, bytes 16-31
//    lo of the same 16 tokens; K-block b = (term b >> 1, page b & 1) takes its scale
//    from lane row + 16 b, i.e. 2^(c_page - m) for hi and 2^(c_page - m - 4) for lo. V is
//    the same LDS rows as K (no second HBM read), gathered transposed with
//    ds_read_b64_tr_b8. l~ comes from one extra MFMA against a tile of ones.
//  * Two barriers per step: (A) step data landed and the previous step fully consumed;
//    (C) P~ and the per-page maxima of the step in LDS.
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

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStepPages = 2;
constexpr int kStepBytes = kStepPages * kPageBytes;    // 36864
constexpr int kStages = 4;
constexpr int kLoadsPerStep = kStepBytes / 1024;       // 36 wave-wide 16-byte loads
constexpr int kChunks = kDQK / 16;                     // 36 chunks of 16 bytes per row
constexpr int kPRow = 144;                             // P~ row: 64 hi, 64 lo, 16 pad
constexpr int kDimTiles = kDV / 16 / kWaves;           // 4 dim tiles per wave
constexpr int kOnesE4M3 = 0x38383838;                  // four E4M3 1.0

template <int NT>
struct __attribute__((aligned(16))) Smem {
  uint8_t pages[kStages][kStepBytes];
  uint8_t ptile[NT * kTileRows * kPRow];
  float2 cl[NT * kTileRows][kStepPages];  // per (row, page): (c, sum of x)
};

__device__ __forceinline__ int rot_of(int n) { return (n >> 2) & 3; }

// s_waitcnt vmcnt(N), leaving the other counters free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most n of this wave's loads are outstanding, rounding n down to a
// supported count (waiting for more is always safe).
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  if (n >= 36) wait_vmcnt<36>();
  else if (n >= 27) wait_vmcnt<27>();
  else if (n >= 18) wait_vmcnt<18>();
  else if (n >= 12) wait_vmcnt<12>();
  else if (n >= 10) wait_vmcnt<10>();
  else if (n >= 9) wait_vmcnt<9>();
  else if (n >= 8) wait_vmcnt<8>();
  else if (n >= 6) wait_vmcnt<6>();
  else if (n >= 5) wait_vmcnt<5>();
  else if (n >= 4) wait_vmcnt<4>();
  else wait_vmcnt<0>();
}

// Workgroup barrier ordering LDS traffic only. __syncthreads() would also fence the
// direct-to-LDS loads still in flight for later stages (vmcnt(0)); their completion is
// awaited per stage with wait_vmcnt before the barrier instead.
__device__ __forceinline__ void block_sync_lds() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wave-wide direct-to-LDS load: lane i's 16 bytes at `gptr` land at LDS byte
// address lds_base + 16 i. Issued from inline asm so that the compiler's wait-count
// pass does not make every later LDS read wait for it (vmcnt(0) would drain the whole
// pipeline). M0 carries the LDS base and is restored afterwards.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  __asm__ volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(base)
      : "memory");
}

__device__ __forceinline__ float ldexp_int(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }

__device__ __forceinline__ v4i ld16(const uint8_t* base, int off) {
  return *(const v4i*)(base + off);
}

__device__ __forceinline__ v8i cat8(v4i a, v4i b) {
  return v8i{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
}

// Map the flat workgroup id to (sorted split index, row block) so that the row blocks
// of one split run on the same XCD (workgroup i goes to XCD i mod 8) and splits are
// dealt round-robin over the XCDs.
__device__ __forceinline__ bool wg_item(const PlanDev& P, int wg, int* part_sorted, int* blk) {
  const int x = wg & 7, k = wg >> 3;
  const int slot = k / P.tiles;
  *blk = k - slot * P.tiles;
  *part_sorted = slot * 8 + x;
  return *part_sorted < P.total_parts;
}

// 2^(a - b) for integer-valued a <= b; 0 when a is -inf.
__device__ __forceinline__ float pow2_diff(float a, float b) {
  return a == -INFINITY ? 0.f : ldexp_int(1.f, (int)(a - b));
}

template <int NT>
__global__ void __launch_bounds__(kThreads, 1)
partial_kernel(const PlanDev P, const uint8_t* __restrict__ q, const uint8_t* __restrict__ kv,
               const int32_t* __restrict__ bt, int64_t bt_stride,
               const int32_t* __restrict__ kv_lens, float scale_log2,
               float* __restrict__ ws_o, float* __restrict__ ws_stats) {
  __shared__ Smem<NT> sm;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;  // lane group: K-block of operands, row group of results
  const int l16 = lane & 15;

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
  const int part = (int)P.part_base[b] + s;
  const int L = min(kv_lens[b], (int)P.kv_len[b]);
  const int chunk_tok = chunk_pages_of(P, b) * kPage;
  const int t0 = s * chunk_tok;
  const int t1 = max(t0, min(t0 + chunk_tok, L));
  const int row0 = blk * NT * kTileRows;  // first row of this work item in its request
  const int32_t* btb = bt + (int64_t)b * bt_stride;

  // ---- roles
  const int qk_rt = w >> 1;        // QK wave: row tile
  const int qk_page = w & 1;       //          page of the step
  const bool is_qk = qk_rt < NT;
  constexpr int kLoaderWaves = 2 * NT < kWaves ? kWaves - 2 * NT : kWaves;
  constexpr int kFirstLoader = 2 * NT < kWaves ? 2 * NT : 0;
  const bool is_loader = w >= kFirstLoader;
  const int li = w - kFirstLoader;  // loader index
  const int my_loads = is_loader ? (kLoadsPerStep - li + kLoaderWaves - 1) / kLoaderWaves : 0;

  // ---- Q^T fragments (QK waves): lane (row l16, group g) holds bytes [32g, 32g + 32)
  // of each 128-byte K-step of its row; the rope step uses groups 0-1 only.
  const int qrow = row0 + qk_rt * kTileRows + l16;
  const bool qrow_valid = is_qk && qrow < P.rows;
  v8i qf[5];
  {
    const uint8_t* qp = q + ((int64_t)b * P.rows + (qrow_valid ? qrow : 0)) * kDQK;
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
    qf[4] = cat8(a, c);
  }
  // causal limit of the QK row: query j sees tokens < L - q_len + j + 1
  const int jq = qrow < P.rows ? qrow / P.heads : P.q_len - 1;
  const int lim_q = min(t1, L - P.q_len + jq + 1);
  // below this token no row of the work item needs a mask
  const int lim_all = min(t1, L - P.q_len + min(row0, P.rows - 1) / P.heads + 1);

  // ---- loader precompute: loader li issues loads k = li, li + LW, ... of every step
  constexpr int kMaxLoads = (kLoadsPerStep + kLoaderWaves - 1) / kLoaderWaves;
  uint32_t ld_off[kMaxLoads];
  uint32_t ld_page[kMaxLoads];
#pragma unroll
  for (int i = 0; i < kMaxLoads; ++i) {
    const int k = min(li + i * kLoaderWaves, kLoadsPerStep - 1);
    const int pg = k / 18, inst = k % 18;
    const int slot = inst * 64 + lane;
    const int n = slot / kChunks, pc = slot % kChunks;
    int c = pc - rot_of(n);
    if (c < 0) c += kChunks;
    ld_off[i] = (uint32_t)(n * kDQK + 16 * c);
    ld_page[i] = (uint32_t)pg;
  }

  const int p_first = t0 / kPage;
  const int p_end = (t1 + kPage - 1) / kPage;
  const int nsteps = t1 > t0 ? (p_end - p_first + kStepPages - 1) / kStepPages : 0;

  auto page_ids = [&](int st, int64_t* ida, int64_t* idb) {
    const int pa = p_first + st * kStepPages;
    const int pb = pa + 1 < p_end ? pa + 1 : pa;  // odd tail: reload page a (never used)
    *ida = btb[pa];
    *idb = btb[pb];
  };
  auto issue = [&](int st, int64_t ida, int64_t idb) {
    const uint8_t* ga = kv + ida * kPageBytes;
    const uint8_t* gb = kv + idb * kPageBytes;
    uint8_t* stage = sm.pages[st % kStages];
#pragma unroll
    for (int i = 0; i < kMaxLoads; ++i) {
      if (i < my_loads) {
        const int k = li + i * kLoaderWaves;
        dma16((ld_page[i] ? gb : ga) + ld_off[i], (uint32_t)(uintptr_t)(LDS_AS uint8_t*)(stage + k * 1024));
      }
    }
  };

  // ---- PV state: rows rt*16 + 4g + jj of every row tile, dims 64w + 16d + l16
  v4f acc[NT][kDimTiles];
  v4f acc1 = v4f{0.f, 0.f, 0.f, 0.f};  // l~ of row tile w (w < NT), ones-tile product
#pragma unroll
  for (int rt = 0; rt < NT; ++rt)
#pragma unroll
    for (int d = 0; d < kDimTiles; ++d) acc[rt][d] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_c[NT][4];   // running max of result rows
  float m_a[NT];      // running max of operand rows (row l16 of each tile)
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // l of rows 4g + jj of row tile w (w < NT)
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
    m_a[rt] = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) m_c[rt][jj] = -INFINITY;
  }

  // transposed V reads: lane (16G + u) names token 16G + 8r + u/2 and the 8-byte half
  // u%2 of a 16-dim chunk; it receives dim 16D + l16 for 8 tokens. V chunks (D < 32)
  // never wrap around the row under the rotation, so each address is base + 16 D.
  int tr_base[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int tokstep = 16 * g + 8 * r + (l16 >> 1);
    const int pg = tokstep >> 5, n = tokstep & 31;
    tr_base[r] = pg * kPageBytes + n * kDQK + 16 * rot_of(n) + 8 * (l16 & 1) + 16 * (kDimTiles * w);
  }
  // K reads of the QK wave: token row n = 16 tt + l16 of its page; chunks 8 c4 + 2g (+1)
  // never wrap for c4 < 4; the rope chunks 32 + 2 (g & 1) (+1) may.
  int k_base[2], k_rope0[2], k_rope1[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int n = 16 * tt + l16;
    const int r = rot_of(n);
    k_base[tt] = qk_page * kPageBytes + n * kDQK + 16 * (2 * g + r);
    int c0 = 32 + 2 * (g & 1) + r, c1 = c0 + 1;
    if (c0 >= kChunks) c0 -= kChunks;
    if (c1 >= kChunks) c1 -= kChunks;
    k_rope0[tt] = qk_page * kPageBytes + n * kDQK + 16 * c0;
    k_rope1[tt] = qk_page * kPageBytes + n * kDQK + 16 * c1;
  }

  wait_vmcnt<0>();  // Q fragments landed; the stage waits below count page loads only
  int64_t nid_a = 0, nid_b = 0;
  if (is_loader) {
    for (int st = 0; st < kStages - 1 && st < nsteps; ++st) {
      int64_t ia, ib;
      page_ids(st, &ia, &ib);
      issue(st, ia, ib);
    }
    if (kStages - 1 < nsteps) page_ids(kStages - 1, &nid_a, &nid_b);
  }

  for (int st = 0; st < nsteps; ++st) {
    if (is_loader) {
      const int issued = min(nsteps, st + kStages - 1);
      wait_vmcnt_at_most((issued - st - 1) * my_loads);
    }
    block_sync_lds();  // (A) step st in LDS; step st - 1 consumed by every wave
    if (is_loader && st + kStages - 1 < nsteps) {
      issue(st + kStages - 1, nid_a, nid_b);
      if (st + kStages < nsteps) page_ids(st + kStages, &nid_a, &nid_b);
    }
    const uint8_t* stage = sm.pages[st % kStages];
    const int tok_step = (p_first + st * kStepPages) * kPage;

    // ---------------- QK^T and softmax of (page qk_page, row tile qk_rt)
    if (is_qk) {
      v4f sacc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        v4f a4 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const v8i kf = cat8(ld16(stage, k_base[tt] + 128 * c4),
                              ld16(stage, k_base[tt] + 128 * c4 + 16));
          a4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[c4], a4, 0, 0, 0, 127, 0, 127);
        }
        v4i ra = ld16(stage, k_rope0[tt]);
        v4i rb = ld16(stage, k_rope1[tt]);
        if (g >= 2) { ra = 0; rb = 0; }
        sacc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat8(ra, rb), qf[4], a4, 0, 0, 0, 127, 0, 127);
      }
      // lane holds S[row l16][token 16 tt + 4g + jj] of the page
      float t[2][4];
      float mx = -INFINITY;
      const int tok_page = tok_step + qk_page * kPage;
      const bool need_mask = tok_page + kPage > lim_all;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float v = sacc[tt][jj] * scale_log2;
          if (need_mask && tok_page + 16 * tt + 4 * g + jj >= lim_q) v = -INFINITY;
          t[tt][jj] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float c = ceilf(mx);                 // -inf when no key of the page is visible
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
      uint8_t* prow = sm.ptile + (qk_rt * kTileRows + l16) * kPRow + qk_page * kPage + 4 * g;
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
      if (g == 0) sm.cl[qk_rt * kTileRows + l16][qk_page] = make_float2(c, xs);
    }
    block_sync_lds();  // (C) P~ and per-page maxima of the step in LDS

    // ---------------- PV for dims [64w, 64w + 64), all row tiles
    {
      // V operand (shared by every row tile): 16 tokens of this lane group per dim tile
      const bool last = st == nsteps - 1;
      v8i vb[kDimTiles];
#pragma unroll
      for (int d = 0; d < kDimTiles; ++d) {
        const v2i b0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(stage + tr_base[0] + 16 * d));
        const v2i b1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS v2i*)(stage + tr_base[1] + 16 * d));
        vb[d] = v8i{b0.x, b0.y, b1.x, b1.y, b0.x, b0.y, b1.x, b1.y};
      }
      if (last) {
        // bytes of tokens past the split's end may be poison: zero them (P~ is 0 there)
        const int valid = t1 - tok_step;  // tokens of this step in range
        uint32_t mk[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          uint32_t m = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (16 * g + 4 * q4 + j < valid) m |= 0xFFu << (8 * j);
          mk[q4] = m;
        }
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d) {
          vb[d][0] &= mk[0]; vb[d][1] &= mk[1]; vb[d][2] &= mk[2]; vb[d][3] &= mk[3];
          vb[d][4] &= mk[0]; vb[d][5] &= mk[1]; vb[d][6] &= mk[2]; vb[d][7] &= mk[3];
        }
      }
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        // per-page maxima of result rows (4g + jj) and operand row (l16)
        bool rescale = false;
        float alpha[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float2 p0 = sm.cl[rt * kTileRows + 4 * g + jj][0];
          const float2 p1 = sm.cl[rt * kTileRows + 4 * g + jj][1];
          const float mn = fmaxf(m_c[rt][jj], fmaxf(p0.x, p1.x));
          alpha[jj] = mn == m_c[rt][jj] ? 1.f : pow2_diff(m_c[rt][jj], mn);
          rescale |= mn != m_c[rt][jj];
          if (rt == w) lsum[jj] = lsum[jj] * alpha[jj] + p0.y * pow2_diff(p0.x, mn) + p1.y * pow2_diff(p1.x, mn);
          m_c[rt][jj] = mn;
        }
        if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
          for (int d = 0; d < kDimTiles; ++d) {
            acc[rt][d][0] *= alpha[0]; acc[rt][d][1] *= alpha[1];
            acc[rt][d][2] *= alpha[2]; acc[rt][d][3] *= alpha[3];
          }
          if (rt == w) {
            acc1[0] *= alpha[0]; acc1[1] *= alpha[1]; acc1[2] *= alpha[2]; acc1[3] *= alpha[3];
          }
        }
        const float2 a0 = sm.cl[rt * kTileRows + l16][0];
        const float2 a1 = sm.cl[rt * kTileRows + l16][1];
        m_a[rt] = fmaxf(m_a[rt], fmaxf(a0.x, a1.x));
        const float cp = (g & 1) ? a1.x : a0.x;
        const int sa = cp == -INFINITY ? 127 : max(0, 127 + (int)(cp - m_a[rt]) - 4 * (g >> 1));
        const uint8_t* prow = sm.ptile + (rt * kTileRows + l16) * kPRow + 16 * g;
        const v8i pa = cat8(ld16(prow, 0), ld16(prow, 64));
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d)
          acc[rt][d] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa, vb[d], acc[rt][d], 0, 0, 0, sa, 0, 127);
        if (rt == w) {
          const v8i ones = v8i{kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3,
                               kOnesE4M3, kOnesE4M3, kOnesE4M3, kOnesE4M3};
          acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pa, ones, acc1, 0, 0, 0, sa, 0, 127);
        }
      }
    }
  }

  // ---------------- write the partials
  const int64_t part_row0 = (int64_t)part * P.rows;
#pragma unroll
  for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = row0 + rt * kTileRows + 4 * g + jj;
      if (row < P.rows) {
        float* orow = ws_o + (part_row0 + row) * kDV + 16 * kDimTiles * w + l16;
#pragma unroll
        for (int d = 0; d < kDimTiles; ++d) orow[16 * d] = acc[rt][d][jj];
        if (rt == w && l16 == 0)
          *(float4*)(ws_stats + (part_row0 + row) * kStatStride) =
              make_float4(m_c[rt][jj], lsum[jj], acc1[jj], 0.f);
      }
    }
  }
}

}  // namespace

int launch_partial(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                   const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                   float softmax_scale, float* ws_o, float* ws_stats, void* stream) {
  const PlanDev& P = plan.dev;
  const int slots = (P.total_parts + 7) / 8;
  const dim3 grid(8 * slots * P.tiles), block(kThreads);
  const float scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t st = (hipStream_t)stream;
  switch (P.nt) {
    case 1: hipLaunchKernelGGL(partial_kernel<1>, grid, block, 0, st, P, q, kv, bt, bt_stride, kv_lens, scale_log2, ws_o, ws_stats); break;
    case 2: hipLaunchKernelGGL(partial_kernel<2>, grid, block, 0, st, P, q, kv, bt, bt_stride, kv_lens, scale_log2, ws_o, ws_stats); break;
    case 3: hipLaunchKernelGGL(partial_kernel<3>, grid, block, 0, st, P, q, kv, bt, bt_stride, kv_lens, scale_log2, ws_o, ws_stats); break;
    default: hipLaunchKernelGGL(partial_kernel<4>, grid, block, 0, st, P, q, kv, bt, bt_stride, kv_lens, scale_log2, ws_o, ws_stats); break;
  }
  return (int)hipGetLastError();
}

}  // namespace mla
