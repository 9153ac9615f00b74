// Merge kernel: combines each row's split partials into BF16 (or fp32) O and fp32 LSE.
//
// Method of TensorRT-LLM PR #20380 "trtllm-gen FMHA: split the KV partials of a row
// across thread groups in fmhaReductionKernel" (Description), re-done for 64-wide
// wavefronts: W workgroups per row (W = 1, 2, 4 or 8, each owning 512 / W of the output
// dims) with G wavefront groups each; group g folds partials g, g + G, ... with the
// online-softmax merge, then the groups are combined through LDS, each scaled by
// 2^(group max - max) and empty groups skipped. A lane owns 8 / W consecutive dims, so
// every partial row is one fully coalesced read of 2 KB / W per wavefront. W = 8 only
// when very few rows hold many splits (one long request): then a workgroup per row
// would leave most CUs idle while each of its waves walks its partials in rounds.
//
// Partials arrive from the split-KV kernel as (m, l, l~, O) with m an integer (log2
// units), so every rescale here is an exact power of two (v_ldexp_f32):
//     M = max_s m_s,  O = sum_s 2^(m_s - M) O_s,  l = sum_s 2^(m_s - M) l_s  (same for l~)
//     out = output_scale * O / l~,   LSE = ln(2) * (M - 8 + log2(l))
// (the 8 undoes the 2^8 scale of the partials' probabilities). A partial with m = -inf
// (a split in which a causal row sees no key) contributes nothing.
//
// Epilogue options (the steps after the combine in the same PR, and the MXFP8 merge
// epilogue of TensorRT-LLM PR #17441 "m3 decode perf clean", commit messages):
//   * sinks: one logit sigma_h per head (units of the scaled scores) joins both sums as
//     2^(sigma_h log2(e) - M + 8); M is first raised to ceil(sigma_h log2 e) when the
//     sink is the larger, so the exact power-of-two rescales still apply. LSE is then
//     the log of the whole denominator.
//   * MXFP8 O: the BF16 values of O, in blocks of 32 consecutive dims, with an E8M0
//     scale 2^e and E4M3 codes of x / 2^e (round to nearest even). The commit messages
//     on the quantize tile and its scale byte 0 fix the two edge cases: e is the
//     smallest integer with amax < 448 * 2^e, strictly (a block whose amax is
//     1.75 * 2^k gets the exponent above 448's), clamped to [-127, 127] and read off
//     the bits of amax with no division; and a block of scale byte 0 (e = -127)
//     saturates: its non-zero elements become +-448, its zeros stay zeros. Four lanes
//     hold one block (8 dims each), so the block max is two lane swaps.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kMaxGroups = 16;
constexpr int kUnroll = 4;

__device__ __forceinline__ float pow2i(float m_from, float m_to) {
  // 2^(m_from - m_to) for integer-valued m_from <= m_to; 0 when m_from is -inf
  return m_from == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.f, (int)(m_from - m_to));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

constexpr float kLog2e = 1.4426950408889634f;

// E8M0 exponent of an MXFP8 block from its amax (a BF16 value, so exact in fp32): the
// smallest e with amax < 448 * 2^e = 1.75 * 2^(e + 8), strictly, clamped to
// [-127, 127]. With amax = f 2^k, f in [1, 2): e = k - 8 when f < 1.75, else k - 7.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ef = (int)((u >> 23) & 0xFF);
  if (ef == 0) return -127;  // zero or below 2^-126: the clamp decides
  const int e = (ef - 127) - 8 + ((u & 0x7FFFFFu) >= 0x600000u ? 1 : 0);
  return min(max(e, -127), 127);
}

// E4M3 code of a block whose scale byte is 0: the block saturates, so a non-zero value
// becomes the largest magnitude (code 0x7E) with its sign and a zero stays a zero.
__device__ __forceinline__ uint32_t mx_saturated_code(float x) {
  const uint32_t u = __float_as_uint(x);
  return ((u >> 24) & 0x80u) | ((u & 0x7FFFFFFFu) != 0u ? 0x7Eu : 0u);
}

// Dynamic shared memory of a merge workgroup, sized by the launch's group count G (a
// workgroup of one wave needs 2 KB, not the 32 KB of 16 groups, so more of them fit on a
// CU): o[G][dims of the slice], then m[G], l[G], l~[G].
inline size_t merge_smem_bytes(int groups, int slices) {
  return (size_t)groups * (size_t)(kDV / slices + 3) * sizeof(float);
}

// kDev: the plan and output_scale come from device memory (graph path).
template <bool kF32Out, bool kDev, int kW>
__global__ void __launch_bounds__(64 * kMaxGroups)
merge_kernel(const PlanDev Parg, const PlanDev* __restrict__ pdev,
             const float* __restrict__ oscale_dev, const float* __restrict__ ws_o,
             const float* __restrict__ ws_stats, float output_scale_arg, void* __restrict__ out,
             float* __restrict__ lse, int groups, const MergeEpilogue ep) {
  extern __shared__ __attribute__((aligned(16))) float merge_smem[];
  const PlanDev& P = kDev ? *pdev : Parg;
  const float output_scale = kDev ? *oscale_dev : output_scale_arg;
  constexpr int kD = 8 / kW;                  // dims per lane
  constexpr int kSlice = kDV / kW;            // dims per workgroup
  float* const so = merge_smem;               // [groups][kSlice]
  float* const sm_m = so + groups * kSlice;
  float* const sm_l = sm_m + groups;
  float* const sm_lt = sm_l + groups;
  // partials in flight per wavefront (4 at W = 1: more registers would halve the
  // workgroups a CU holds, which costs more than the extra loads give)
  constexpr int kU = kW >= 2 ? 16 : 4;
  // groups in use: the launch's, or the device plan's (<= the launch's) on the graph path
  const int G = kDev ? min(P.groups, groups) : groups;
  const int row_global = blockIdx.x / kW;  // (b * q_len + j) * H + h
  const int dim0 = (blockIdx.x - row_global * kW) * kSlice;
  const int b = row_global / P.rows;
  const int r = row_global - b * P.rows;
  const int S = P.splits[b];
  const int base = (int)P.part_base[b];
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  float M = -INFINITY, l = 0.f, lt = 0.f;
  float o[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) o[i] = 0.f;
  for (int s0 = gw; gw < G && s0 < S; s0 += kU * G) {
    float4 stv[kU];
    float a[kU][kD];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int s = s0 + u * G;
      if (s < S) {
        const int64_t pr = (int64_t)(base + s) * P.rows + r;
        stv[u] = *(const float4*)(ws_stats + pr * kStatStride);
        const float* op = ws_o + pr * kDV + dim0 + kD * lane;
        if constexpr (kD == 8) {
          const float4 x = ((const float4*)op)[0], y = ((const float4*)op)[1];
          a[u][0] = x.x; a[u][1] = x.y; a[u][2] = x.z; a[u][3] = x.w;
          a[u][4] = y.x; a[u][5] = y.y; a[u][6] = y.z; a[u][7] = y.w;
        } else if constexpr (kD == 4) {
          const float4 x = *(const float4*)op;
          a[u][0] = x.x; a[u][1] = x.y; a[u][2] = x.z; a[u][3] = x.w;
        } else if constexpr (kD == 2) {
          const float2 x = *(const float2*)op;
          a[u][0] = x.x; a[u][1] = x.y;
        } else {
          a[u][0] = *op;
        }
      } else {
        stv[u] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
#pragma unroll
        for (int i = 0; i < kD; ++i) a[u][i] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float ms = stv[u].x;
      if (ms == -INFINITY) continue;
      const float Mn = fmaxf(M, ms);
      const float wa = pow2i(M, Mn), wb = pow2i(ms, Mn);
#pragma unroll
      for (int i = 0; i < kD; ++i) o[i] = o[i] * wa + a[u][i] * wb;
      l = l * wa + stv[u].y * wb;
      lt = lt * wa + stv[u].z * wb;
      M = Mn;
    }
  }
#pragma unroll
  for (int i = 0; i < kD; ++i) so[gw * kSlice + kD * lane + i] = o[i];
  if (lane == 0) {
    sm_m[gw] = M;
    sm_l[gw] = l;
    sm_lt[gw] = lt;
  }
  __syncthreads();

  float Mx = -INFINITY;
  for (int k = 0; k < G; ++k) Mx = fmaxf(Mx, sm_m[k]);
  // a sink above every partial's max raises M to its (integer) ceiling
  const float sig = ep.sinks != nullptr ? ep.sinks[r % P.heads] * kLog2e : -INFINITY;
  if (sig > Mx) Mx = ceilf(sig);
  float wk[kMaxGroups];
  float L = 0.f, Lt = 0.f;
  for (int k = 0; k < G; ++k) {
    wk[k] = Mx == -INFINITY ? 0.f : pow2i(sm_m[k], Mx);
    L += wk[k] * sm_l[k];
    Lt += wk[k] * sm_lt[k];
  }
  if (sig > -INFINITY) {
    const float ps = exp2f(sig - Mx + 8.f);
    L += ps;
    Lt += ps;
  }
  const float inv = Lt > 0.f ? output_scale / Lt : 0.f;
  if (kF32Out || ep.o_fp8 == nullptr) {
    for (int d = threadIdx.x; d < kSlice; d += blockDim.x) {
      float acc = 0.f;
      for (int k = 0; k < G; ++k) acc += wk[k] * so[k * kSlice + d];
      const float v = acc * inv;
      if (kF32Out)
        ((float*)out)[(int64_t)row_global * kDV + dim0 + d] = v;
      else
        ((uint16_t*)out)[(int64_t)row_global * kDV + dim0 + d] = f32_to_bf16_rne(v);
    }
  } else if (threadIdx.x < kSlice / 8) {
    // MXFP8 (and BF16 when out is given): lane t owns dims dim0 + 8t .. dim0 + 8t + 7
    const int dl = 8 * (int)threadIdx.x;  // in the slice (so)
    const int d0 = dim0 + dl;             // in the row
    float vb[8];
    uint32_t hw[4];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = 0.f;
      for (int k = 0; k < G; ++k) acc += wk[k] * so[k * kSlice + dl + i];
      const uint16_t h16 = f32_to_bf16_rne(acc * inv);
      vb[i] = __uint_as_float((uint32_t)h16 << 16);
      amax = fmaxf(amax, fabsf(vb[i]));
      if (i & 1)
        hw[i >> 1] |= (uint32_t)h16 << 16;
      else
        hw[i >> 1] = h16;
    }
    if (out != nullptr)
      *(uint4*)((uint16_t*)out + (int64_t)row_global * kDV + d0) =
          make_uint4(hw[0], hw[1], hw[2], hw[3]);
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int e = mx_block_exponent(amax);
    int c0 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(vb[0], -e),
                                             __builtin_amdgcn_ldexpf(vb[1], -e), 0, false);
    c0 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(vb[2], -e),
                                         __builtin_amdgcn_ldexpf(vb[3], -e), c0, true);
    int c1 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(vb[4], -e),
                                             __builtin_amdgcn_ldexpf(vb[5], -e), 0, false);
    c1 = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(vb[6], -e),
                                         __builtin_amdgcn_ldexpf(vb[7], -e), c1, true);
    if (e == -127) {  // scale byte 0 (uniform over the block's four lanes)
      uint32_t s0 = 0, s1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s0 |= mx_saturated_code(vb[i]) << (8 * i);
        s1 |= mx_saturated_code(vb[4 + i]) << (8 * i);
      }
      c0 = (int)s0;
      c1 = (int)s1;
    }
    *(uint2*)(ep.o_fp8 + (int64_t)row_global * kDV + d0) = make_uint2((uint32_t)c0, (uint32_t)c1);
    if ((threadIdx.x & 3) == 0)
      ep.o_fp8_scales[(int64_t)row_global * (kDV / 32) + (d0 >> 5)] = (uint8_t)(e + 127);
  }
  if (lse != nullptr && dim0 == 0 && threadIdx.x == 0)
    lse[row_global] = L > 0.f ? 0.69314718055994531f * ((Mx - 8.f) + log2f(L)) : -INFINITY;
}

// Fold of cooperative splits (plans whose dev.subs > 1 run a split on several
// workgroups, each over its own run of the split's keys): the partial state of (split p,
// row r) from its sub-ranges' states by the combine above without the final division,
//     M = max_i m_i,  O = sum_i 2^(m_i - M) O_i,  l = sum_i 2^(m_i - M) l_i  (same for l~),
// in sub-range order. One wavefront per (split, row); lane i owns dims [8 i, 8 i + 8).
__global__ void __launch_bounds__(256)
fold_kernel(int n, int rows, int subs, const PlanDev* __restrict__ pdev,
            const float* __restrict__ sub_o, const float* __restrict__ sub_stats,
            float* __restrict__ o, float* __restrict__ stats) {
  const int w = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  // graph plans: the launch covers the capacity, the device plan the splits that exist
  if (w >= n || (pdev != nullptr && w >= pdev->total_parts * rows)) return;
  const int lane = threadIdx.x & 63;
  const int p = w / rows, r = w - p * rows;
  const int64_t k0 = (int64_t)p * subs * rows + r;  // slot of (p, sub 0, r); sub i: + i rows
  float M = -INFINITY;
  for (int i = 0; i < subs; ++i) M = fmaxf(M, sub_stats[(k0 + (int64_t)i * rows) * kStatStride]);
  float l = 0.f, lt = 0.f;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  for (int i = 0; i < subs; ++i) {
    const int64_t k = k0 + (int64_t)i * rows;
    const float4 st = *(const float4*)(sub_stats + k * kStatStride);
    const float wt = pow2i(st.x, M);
    if (wt == 0.f) continue;  // a sub-range without a visible key (wave-uniform)
    l += wt * st.y;
    lt += wt * st.z;
    const float4* src = (const float4*)(sub_o + k * kDV + 8 * lane);
    const float4 x = src[0], y = src[1];
    a.x += wt * x.x; a.y += wt * x.y; a.z += wt * x.z; a.w += wt * x.w;
    b.x += wt * y.x; b.y += wt * y.y; b.z += wt * y.z; b.w += wt * y.w;
  }
  float4* dst = (float4*)(o + ((int64_t)p * rows + r) * kDV + 8 * lane);
  dst[0] = a;
  dst[1] = b;
  if (lane == 0)
    *(float4*)(stats + ((int64_t)p * rows + r) * kStatStride) = make_float4(M, l, lt, 0.f);
}

}  // namespace

int launch_fold(const mla_decode_plan_s& plan, const float* sub_o, const float* sub_stats,
                float* o, float* stats, void* stream, const DeviceArgs* dev) {
  const PlanDev& P = plan.dev;
  const int n = P.total_parts * P.rows;  // graph plans: the capacity
  if (n == 0) return 0;
  hipLaunchKernelGGL(fold_kernel, dim3((n + 3) / 4), dim3(256), 0, (hipStream_t)stream, n,
                     P.rows, P.subs, dev ? dev->plan : nullptr, sub_o, sub_stats, o, stats);
  return (int)hipGetLastError();
}

int launch_merge(const mla_decode_plan_s& plan, const float* ws_o, const float* ws_stats,
                 float output_scale, void* o, bool o_is_f32, float* lse, void* stream,
                 const DeviceArgs* dev, const MergeEpilogue* epi) {
  const PlanDev& P = plan.dev;
  const int rows_total = P.batch * P.rows;
  const int groups = plan.merge_groups;
  const PlanDev* pd = dev ? dev->plan : nullptr;
  const float* od = dev ? dev->output_scale : nullptr;
  const MergeEpilogue ep = epi ? *epi : MergeEpilogue{nullptr, nullptr, nullptr};
  hipStream_t st = (hipStream_t)stream;
  const int W = plan.merge_slices;
  const dim3 grid(rows_total * W), block(64 * groups);
  // one instantiation per (output type, plan source, slices)
#define MLA_MERGE_LAUNCH(F32, DEV, KW) \
  hipLaunchKernelGGL((merge_kernel<F32, DEV, KW>), grid, block, merge_smem_bytes(groups, KW), st, P, pd, od, ws_o, ws_stats, output_scale, o, lse, groups, ep)
#define MLA_MERGE_W(F32, DEV)                      \
  switch (W) {                                     \
    case 1: MLA_MERGE_LAUNCH(F32, DEV, 1); break;  \
    case 2: MLA_MERGE_LAUNCH(F32, DEV, 2); break;  \
    case 4: MLA_MERGE_LAUNCH(F32, DEV, 4); break;  \
    default: MLA_MERGE_LAUNCH(F32, DEV, 8); break; \
  }
  if (o_is_f32) {
    if (dev) { MLA_MERGE_W(true, true) } else { MLA_MERGE_W(true, false) }
  } else {
    if (dev) { MLA_MERGE_W(false, true) } else { MLA_MERGE_W(false, false) }
  }
#undef MLA_MERGE_W
#undef MLA_MERGE_LAUNCH
  return (int)hipGetLastError();
}

}  // namespace mla
