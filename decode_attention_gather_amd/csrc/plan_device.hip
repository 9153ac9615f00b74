// Device split planner for the graph path of split-KV MLA decode.
//
// The same plan as the host planner (plan.cpp), computed on the GPU from the request
// lengths in device memory, so that planning, the partial kernel and the merge can be
// captured in one HIP graph and replayed while the lengths change. This is the setting
// of TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA decode slower after #19338" (follow-up
// comments: under CUDA graphs the KV lengths are not on the host, so the split plan is
// made from device data and the kernel skips empty splits).
//
// One workgroup of 256 threads; thread b owns request b:
//   L_b = clamp(kv_lens[b], 0, max_kv_len), pages_b = ceil(L_b / 32)
//   wanted splits: the uniform bound min(split_kv, cap), or the one-wave proportional
//   rule clamp(ceil(pages_b / C), 1, cap) with C the smallest split length for which
//   the sum of those fits the host planner's XCD-aware split budget (the same integer
//   search as the host planner)
//   S_b = clamp(wanted, 1, max(pages_b, 1)), at least ceil(pages_b / 65535),
//   chunk_b = ceil(pages_b / S_b) pages, S_b = ceil(pages_b / chunk_b)  (no empty split)
// then the requests are ranked longest chunk first (ties by index, the host planner's
// stable order) and the prefix sums of S_b give each request's first split and the
// sorted work list. A request of length 0 gets one split with no keys (its rows come
// out with O = 0 and LSE = -inf).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kPlanThreads = 256;
static_assert(kPlanThreads >= kMaxBatch, "one thread per request");

__device__ __forceinline__ int32_t wave_sum(int32_t v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ long long wave_sum64(long long v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
constexpr int kPlanWaves = kPlanThreads / 64;

struct PlanParams {
  int32_t batch, q_len, heads, rows, tiles, nt;
  int32_t max_kv_len, split_kv, max_split_kv, num_cus, cap_parts, max_groups;
  int32_t budget;  // splits that fill the chip once
};

__global__ void __launch_bounds__(kPlanThreads)
device_plan_kernel(const PlanParams pp, const int32_t* __restrict__ kv_lens,
                   PlanDev* __restrict__ out) {
  __shared__ int32_t s_splits[kMaxBatch];
  __shared__ int32_t s_chunk[kMaxBatch];
  __shared__ int32_t s_order[kMaxBatch];
  // per-wave partial results (wave reductions, then one pass over the 4 waves: no
  // contended LDS atomics)
  __shared__ int32_t s_part[kPlanWaves];
  __shared__ int32_t s_pmax[kPlanWaves];
  __shared__ long long s_psum[kPlanWaves];
  __shared__ int32_t s_smax[kPlanWaves];
  __shared__ int32_t s_wpart[5][kPlanWaves];  // sum_b rows min(16 >> k, S_b), k = 0..4
  const int b = threadIdx.x;
  const bool live = b < pp.batch;

  int32_t L = 0;
  if (live) L = min(max(kv_lens[b], 0), pp.max_kv_len);
  const int64_t pages = ((int64_t)L + kPage - 1) / kPage;
  {
    const int32_t pm = wave_max(live ? (int32_t)pages : 1);   // pages <= 2^26
    const long long ps = wave_sum64(live ? pages : 0);        // up to 64 x 2^26
    if ((b & 63) == 0) {
      s_pmax[b >> 6] = pm;
      s_psum[b >> 6] = ps;
    }
  }
  __syncthreads();
  int64_t total_pages = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) total_pages += s_psum[w];

  // proportional plan: the smallest split length C (pages) with
  // sum_b clamp(ceil(pages_b / C), 1, cap) <= budget; every thread runs the same search
  int64_t C = 1;
  if (pp.split_kv <= 0) {
    const int64_t Bn = pp.batch, budget = pp.budget;
    int32_t maxp = 1;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) maxp = max(maxp, s_pmax[w]);
    int64_t lo = 1, hi = maxp;
    if (budget > Bn) hi = min(hi, (total_pages + (budget - Bn) - 1) / (budget - Bn));
    else lo = hi;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;  // <= max pages < 2^27: 32-bit division
      const uint32_t p32 = (uint32_t)pages, m32 = (uint32_t)mid;
      int32_t n = live ? (int32_t)min(max((p32 + m32 - 1u) / m32, 1u), (uint32_t)pp.max_split_kv)
                       : 0;
      n = wave_sum(n);
      if ((b & 63) == 0) s_part[b >> 6] = n;
      __syncthreads();
      int64_t tot = 0;
#pragma unroll
      for (int w = 0; w < kPlanWaves; ++w) tot += s_part[w];
      __syncthreads();
      if (tot <= budget) hi = mid; else lo = mid + 1;
    }
    C = lo;
  }

  if (live) {
    int64_t want;
    if (pp.split_kv > 0) {
      want = min(pp.split_kv, pp.max_split_kv);
    } else {
      want = max((int64_t)1, min((pages + C - 1) / C, (int64_t)pp.max_split_kv));
    }
    // pages < 2^27 and s <= pages: 32-bit divisions
    const uint32_t p32 = (uint32_t)pages;
    uint32_t s = (uint32_t)max((int64_t)1, min(want, max(pages, (int64_t)1)));
    s = max(s, (p32 + kMaxChunkPages - 1u) / kMaxChunkPages);
    const uint32_t chunk = max(1u, (p32 + s - 1u) / s);
    s = max(1u, (p32 + chunk - 1u) / chunk);
    s_splits[b] = (int32_t)s;
    s_chunk[b] = (int32_t)chunk;
    out->kv_len[b] = (uint32_t)L;
    out->splits[b] = (uint16_t)s;
  }
  {
    const int32_t sb = live ? s_splits[b] : 0;
    const int32_t sm = wave_max(sb);
    int32_t wv[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) wv[k] = wave_sum(pp.rows * min(16 >> k, sb));  // <= 2^22 each
    if ((b & 63) == 0) {
      s_smax[b >> 6] = sm;
#pragma unroll
      for (int k = 0; k < 5; ++k) s_wpart[k][b >> 6] = wv[k];
    }
  }
  __syncthreads();
  if (live) {
    int32_t base = 0, rank = 0;
    for (int i = 0; i < pp.batch; ++i) {
      if (i < b) base += s_splits[i];
      if (s_chunk[i] > s_chunk[b] || (s_chunk[i] == s_chunk[b] && i < b)) ++rank;
    }
    out->part_base[b] = (uint32_t)base;
    s_order[rank] = b;
  }
  __syncthreads();
  if (live) {
    uint32_t run = 0;
    for (int e = 0; e <= b; ++e) run += (uint32_t)s_splits[s_order[e]];
    out->sorted[b] = (run << 8) | (uint32_t)s_order[b];
    if (b == pp.batch - 1) {
      out->batch = pp.batch;
      out->q_len = pp.q_len;
      out->heads = pp.heads;
      out->rows = pp.rows;
      out->tiles = pp.tiles;
      // never more work items than the launches were sized for (the host bound holds by
      // construction; the clamp only keeps a broken bound from reading past them)
      out->total_parts = (int32_t)min(run, (uint32_t)pp.cap_parts);
      out->nt = pp.nt;
      // merge width by the host planner's rule, from the actual splits
      int32_t s_max = 0;
      long long s_waves[5] = {0, 0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < kPlanWaves; ++w) {
        s_max = max(s_max, s_smax[w]);
#pragma unroll
        for (int k = 0; k < 5; ++k) s_waves[k] += s_wpart[k][w];
      }
      int32_t g = 1;
      while (g * 2 <= 16 && g * 2 <= s_max) g *= 2;
      auto waves = [&](int32_t gg) { return s_waves[__builtin_ctz(16 / gg)]; };
      while (g > 1 && waves(g) > (long long)kMergeWavesPerCu * pp.num_cus) g /= 2;
      out->groups = min(g, pp.max_groups);
    }
  }
}

}  // namespace

int launch_device_plan(const mla_decode_plan_s& plan, const int32_t* kv_lens, PlanDev* out,
                       void* stream) {
  const PlanDev& d = plan.dev;
  PlanParams pp;
  pp.batch = d.batch;
  pp.q_len = d.q_len;
  pp.heads = d.heads;
  pp.rows = d.rows;
  pp.tiles = d.tiles;
  pp.nt = d.nt;
  pp.max_kv_len = plan.max_kv_len;
  pp.split_kv = plan.split_kv;
  pp.max_split_kv = plan.max_split_kv;
  pp.num_cus = plan.num_cus;
  pp.cap_parts = d.total_parts;
  pp.max_groups = plan.merge_groups;
  pp.budget = (int32_t)split_budget(plan.num_cus, d.tiles);
  hipLaunchKernelGGL(device_plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream,
                     pp, kv_lens, out);
  return (int)hipGetLastError();
}

}  // namespace mla
