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

// Sum over the 64 lanes, every lane receiving it: row rotations by 8, 4, 2, 1 (DPP)
// sum each 16-lane row, then the VALU lane swaps add lanes l ^ 32 and l ^ 16. No LDS
// round trip, unlike a shuffle chain: this sum sits on the planner's critical path, once
// per step of its binary search. All 64 lanes must be active.
__device__ __forceinline__ int32_t wave_sum(int32_t v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);  // row_ror:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x122, 0xF, 0xF, false);  // row_ror:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x121, 0xF, 0xF, false);  // row_ror:1
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = (int32_t)(a[0] + a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return (int32_t)(b[0] + b[1]);
}
__device__ __forceinline__ long long wave_sum64(long long v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {  // as wave_sum, with max
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x122, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x121, 0xF, 0xF, false));
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max((int32_t)a[0], (int32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((int32_t)b[0], (int32_t)b[1]);
}
constexpr int kPlanWaves = kPlanThreads / 64;

// Inclusive prefix sum over the 64 lanes (lane l receives the sum of lanes 0..l): row
// shifts by 1, 2, 4, 8 within each 16-lane row, then the last lane of row 0 added to
// rows 1-3 and that of row 1 to rows 2-3 (DPP row broadcasts). All lanes must be active.
__device__ __forceinline__ uint32_t wave_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

struct PlanParams {
  int32_t batch, q_len, heads, rows, tiles, nt;
  int32_t max_kv_len, split_kv, max_split_kv, num_cus, cap_parts, max_groups;
  int32_t budget;  // splits that fill the chip once
  int32_t subs;    // workgroups per (split, row block), decided by the host
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
  // Up to 64 requests, every wave holds all of them (lane = request) and reduces and
  // searches on its own, with no barrier; beyond that the waves' sums meet in LDS. All
  // sums are of integers, so both ways give the same plan.
  const bool one_wave = pp.batch <= 64;
  const int lane = b & 63;
  uint32_t ps32 = (uint32_t)pages;  // pages of the request this lane searches with
  bool s_live = live;
  if (one_wave) {
    s_live = lane < pp.batch;
    const int32_t Ll = s_live ? min(max(kv_lens[lane], 0), pp.max_kv_len) : 0;
    ps32 = (uint32_t)(((int64_t)Ll + kPage - 1) / kPage);
  }
  int64_t total_pages = 0;
  int32_t maxp = 1;
  if (one_wave) {
    // pages <= 2^26: the low and high 16 bits summed apart cannot overflow 32 bits
    maxp = max(1, wave_max(s_live ? (int32_t)ps32 : 1));
    const uint32_t lo16 = (uint32_t)wave_sum((int32_t)(ps32 & 0xFFFFu));
    const uint32_t hi16 = (uint32_t)wave_sum((int32_t)(ps32 >> 16));
    total_pages = (int64_t)lo16 + ((int64_t)hi16 << 16);
  } else {
    const int32_t pm = wave_max(live ? (int32_t)pages : 1);   // pages <= 2^26
    const long long ps = wave_sum64(live ? pages : 0);        // up to 64 x 2^26
    if ((b & 63) == 0) {
      s_pmax[b >> 6] = pm;
      s_psum[b >> 6] = ps;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
      total_pages += s_psum[w];
      maxp = max(maxp, s_pmax[w]);
    }
  }

  // proportional plan: the smallest split length C (pages) with
  // sum_b clamp(ceil(pages_b / C), 1, cap) <= budget; every thread runs the same search
  int64_t C = 1;
  if (pp.split_kv <= 0) {
    const int64_t Bn = pp.batch, budget = pp.budget;
    int64_t lo = 1, hi = maxp;
    if (budget > Bn) hi = min(hi, (total_pages + (budget - Bn) - 1) / (budget - Bn));
    else lo = hi;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;  // <= max pages < 2^27: 32-bit division
      const uint32_t m32 = (uint32_t)mid;
      int32_t n = s_live ? (int32_t)min(max((ps32 + m32 - 1u) / m32, 1u), (uint32_t)pp.max_split_kv)
                         : 0;
      n = wave_sum(n);
      int64_t tot = n;
      if (!one_wave) {
        if ((b & 63) == 0) s_part[b >> 6] = n;
        __syncthreads();
        tot = 0;
#pragma unroll
        for (int w = 0; w < kPlanWaves; ++w) tot += s_part[w];
        __syncthreads();
      }
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
  if (pp.batch <= 64) {
    if (b < 64) {  // wave 0 holds every request: bases by a scan, ranks by lane reads
      const int32_t sb = live ? s_splits[b] : 0;
      const int32_t cb = live ? s_chunk[b] : 0;
      const int32_t base = (int32_t)wave_scan((uint32_t)sb) - sb;
      int32_t rank = 0;
      for (int i = 0; i < pp.batch; ++i) {
        const int32_t ci = __builtin_amdgcn_readlane(cb, i);
        rank += (ci > cb || (ci == cb && i < b)) ? 1 : 0;
      }
      if (live) {
        out->part_base[b] = (uint32_t)base;
        s_order[rank] = b;
      }
    }
  } else if (live) {
    int32_t base = 0, rank = 0;
    for (int i = 0; i < pp.batch; ++i) {
      if (i < b) base += s_splits[i];
      if (s_chunk[i] > s_chunk[b] || (s_chunk[i] == s_chunk[b] && i < b)) ++rank;
    }
    out->part_base[b] = (uint32_t)base;
    s_order[rank] = b;
  }
  __syncthreads();
  // running split count along the issue order: one wave-wide inclusive scan when the
  // batch fits in wave 0, else a walk over the order
  uint32_t run = 0;
  if (pp.batch <= 64) {
    if (b < 64) run = wave_scan((uint32_t)(live ? s_splits[s_order[b]] : 0));
  } else if (live) {
    for (int e = 0; e <= b; ++e) run += (uint32_t)s_splits[s_order[e]];
  }
  if (live) {
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
      out->subs = pp.subs;
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
  pp.subs = d.subs;
  hipLaunchKernelGGL(device_plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)stream,
                     pp, kv_lens, out);
  return (int)hipGetLastError();
}

}  // namespace mla
