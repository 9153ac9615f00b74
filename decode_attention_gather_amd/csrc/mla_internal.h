// Internal types shared by the planner, the C-ABI layer and the two kernels of
// libmla_decode.so. Not installed; the public interface is include/mla_decode.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

#ifndef __HIPCC__
#define __host__
#define __device__
#endif

namespace mla {

constexpr int kDQK = MLA_D_QK;             // 576 bytes per cached row
constexpr int kDV = MLA_D_V;               // 512 latent = V = O width
constexpr int kPage = MLA_PAGE_SIZE;       // 32 tokens per page
constexpr int kPageBytes = kPage * kDQK;   // 18432
constexpr int kTileRows = 16;              // query rows per MFMA row tile
constexpr int kMaxTilesPerBlock = 2;       // narrow kernel: row tiles per workgroup
constexpr int kWideMaxTiles = 6;           // wide kernel: 4 or 6 row tiles (96 rows)
constexpr int kMaxBatch = MLA_MAX_BATCH;
constexpr int kMaxChunkPages = 65535;      // split length limit (fits uint16)
constexpr int kStatStride = 4;             // (m, l, l~, 0) per (split, row)
constexpr int kMergeWavesPerCu = 32;      // merge launch budget: waves resident per CU
constexpr int kMaxMergeSlices = 8;         // merge: at most 8 workgroups per row
constexpr int kMaxSubs = 8;                // workgroups sharing one split (small grids)
constexpr int kMinSubSteps = 2;            // 2-page steps per workgroup when shared
constexpr int kXcds = 8;                   // XCDs of an MI355X; workgroup i runs on XCD i mod 8

// Everything the kernels need from a plan, passed by value as a kernel argument
// (3.6 KB, under the 4 KB kernel-argument limit). Requests are issued longest split
// first: sorted entry e holds (running split count through e) << 8 | request id.
// Pages per split of request b are ceil(ceil(kv_len[b] / 32) / splits[b]); the kernels
// clamp every key range to the plan's kv_len, so a larger device length cannot make
// them read past the block-table row the plan was checked against.
struct PlanDev {
  int32_t batch;
  int32_t q_len;
  int32_t heads;
  int32_t rows;         // q_len * heads, rows per request
  int32_t tiles;        // row blocks (workgroups) per split: ceil(rows / (16 nt))
  int32_t total_parts;  // sum of splits
  int32_t nt;           // 16-row tiles per row block: 1, 2 (narrow) or 4, 6 (wide)
  int32_t groups;       // merge: wavefront groups per row (<= the launch's groups)
  int32_t subs;         // workgroups per (split, row block): 1, or more on a small grid
  uint32_t sorted[kMaxBatch];     // (part_end << 8) | request
  uint32_t kv_len[kMaxBatch];     // per request: the plan's (host) length
  uint32_t part_base[kMaxBatch];  // per request: index of its first split
  uint16_t splits[kMaxBatch];     // per request
};
static_assert(sizeof(PlanDev) <= 3800, "kernel argument budget");

__host__ __device__ inline int chunk_pages_of(const PlanDev& P, int b) {
  const int pages = (int)((P.kv_len[b] + kPage - 1) / kPage);
  return (pages + P.splits[b] - 1) / P.splits[b];
}

// Keys [*t0, *t1) of split s of request b, whose length (already clamped to the plan's)
// is L: the split's whole pages cut to [0, L) and, with key windows (kv_bounds: int32
// [B][2], the window [start_b, end_b) of issue #20510's kv_bounds argument), to the
// window. An empty range has *t1 == *t0.
__host__ __device__ inline void split_keys(const PlanDev& P, int b, int s, int L,
                                           const int32_t* kv_bounds, int* t0, int* t1) {
  const int chunk = chunk_pages_of(P, b) * kPage;
  int lo = s * chunk;
  int hi = lo + chunk < L ? lo + chunk : L;
  if (kv_bounds != nullptr) {
    const int wlo = kv_bounds[2 * b], whi = kv_bounds[2 * b + 1];
    lo = wlo > lo ? wlo : lo;
    hi = whi < hi ? whi : hi;
  }
  *t0 = lo;
  *t1 = hi > lo ? hi : lo;
}

// Flat workgroup id -> work item (sorted split index ps, sub-range sub, row block blk).
// The row blocks of one (split, sub) run on one XCD (workgroup i goes to XCD i mod 8)
// and (split, sub) pairs are dealt round-robin over the XCDs. False past the last item.
__host__ __device__ inline bool work_item(const PlanDev& P, int wg, int* ps, int* sub,
                                          int* blk) {
  const int x = wg & 7, k = wg >> 3;
  const int slot = k / P.tiles;
  *blk = k - slot * P.tiles;
  const int v = slot * 8 + x;
  *ps = v / P.subs;
  *sub = v - *ps * P.subs;
  return v < P.total_parts * P.subs;
}

// Keys of sub-range sub of a split's keys [*t0, *t1) when P.subs workgroups share the
// split: the split's pages, counted from its first, cut into P.subs runs of whole
// 2-page steps (ceil(steps / subs) each; trailing runs may be empty). An empty run is
// the empty range at the split's end.
__host__ __device__ inline void sub_keys(const PlanDev& P, int sub, int* t0, int* t1) {
  if (P.subs <= 1 || *t1 <= *t0) return;
  const int pf = *t0 / kPage, pe = (*t1 + kPage - 1) / kPage;
  const int per = ((pe - pf + 1) / 2 + P.subs - 1) / P.subs;  // steps per run
  const int lo = (pf + 2 * per * sub) * kPage, hi = (pf + 2 * per * (sub + 1)) * kPage;
  const int a = lo > *t0 ? lo : *t0, b = hi < *t1 ? hi : *t1;
  if (b > a) {
    *t0 = a;
    *t1 = b;
  } else {
    *t0 = *t1;
  }
}

}  // namespace mla

// Host-side plan object (opaque to callers). A graph plan (device_lengths != 0) holds
// capacities only: the request lengths stay on the device, a planner kernel writes the
// PlanDev into the head of the workspace on every call, and dev.total_parts is the
// capacity the launches are sized for.
struct mla_decode_plan_s {
  mla::PlanDev dev;
  int32_t device_lengths;
  int32_t kv_dtype;       // MLA_KV_E4M3 or MLA_KV_BF16
  int32_t max_kv_len;     // graph plans: upper bound of every device length
  int32_t split_kv;       // graph plans: the uniform bound, 0 = proportional planner
  int32_t max_split_kv;   // graph plans: per-request split cap
  size_t ws_plan_bytes;   // graph plans: device PlanDev at the head of the workspace
  int32_t merge_groups;
  int32_t merge_slices;   // workgroups per row in the merge (1, 2, 4 or 8 dim slices)
  int32_t max_splits;
  int32_t num_cus;
  size_t ws_o_bytes;      // fp32 partial O region
  size_t ws_stats_bytes;  // fp32 (m, l, l~, 0) region
  size_t ws_sub_o_bytes;      // dev.subs > 1: the sub-ranges' fp32 O, after the stats
  size_t ws_sub_stats_bytes;  // dev.subs > 1: their (m, l, l~, 0), after that
  int32_t* kv_lens;       // host copy [batch]
};

namespace mla {

// A grid of fewer workgroups than CUs (graph plans: by capacity). Such grids leave
// CUs idle, and each busy CU must pull more bytes per second: kernels keep more loads
// in flight per workgroup there.
inline bool narrow_underfilled(const mla_decode_plan_s& plan) {
  return (int64_t)plan.dev.total_parts * plan.dev.subs * plan.dev.tiles <
         (int64_t)plan.num_cus;
}

// Workspace carve-up (256-byte aligned regions): [device plan (graph plans)] partial O,
// stats, and with dev.subs > 1 the sub-ranges' O and stats.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t workspace_bytes_of(const mla_decode_plan_s& plan) {
  return plan.ws_plan_bytes + plan.ws_o_bytes + plan.ws_stats_bytes + plan.ws_sub_o_bytes +
         plan.ws_sub_stats_bytes;
}

// Graph path: where the kernels find the plan and the scales (device memory).
struct DeviceArgs {
  const PlanDev* plan;
  const float* softmax_scale;
  const float* output_scale;
};

// Launchers (defined next to their kernels). Return a hipError_t value as int. With
// dev != nullptr the kernels read the plan and the scales from device memory and the
// launch is sized by the plan's capacity. q_lens (device, may be null): per-request
// query tokens of a ragged batch, each clamped to [0, q_len]. kv_bounds (device, may be
// null): per-request key windows [start, end), int32 [B][2].
int launch_partial(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                   const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                   float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                   const DeviceArgs* dev = nullptr, const int32_t* q_lens = nullptr,
                   const int32_t* kv_bounds = nullptr);
// BF16 cache (rows of 576 BF16 values), blocks of 1 or 2 row tiles.
int launch_partial_bf16(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                        const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                        float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                        const DeviceArgs* dev, const int32_t* q_lens, const int32_t* kv_bounds);
// BF16 cache, blocks of 4 or 6 row tiles.
int launch_partial_bf16_wide(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                             const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                             float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                             const DeviceArgs* dev, const int32_t* q_lens,
                             const int32_t* kv_bounds);
int launch_partial_wide(const mla_decode_plan_s& plan, const uint8_t* q, const uint8_t* kv,
                        const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                        float softmax_scale, float* ws_o, float* ws_stats, void* stream,
                        const DeviceArgs* dev, const int32_t* q_lens, const int32_t* kv_bounds);
// Optional steps of the merge epilogue (any pointer may be null): per-head sink logits
// (fp32 [H]), and the MXFP8 form of O (E4M3 codes [rows][512], E8M0 scales [rows][16];
// both or neither). With o_fp8 set, o (BF16) may be null.
struct MergeEpilogue {
  const float* sinks;
  uint8_t* o_fp8;
  uint8_t* o_fp8_scales;
};
int launch_merge(const mla_decode_plan_s& plan, const float* ws_o, const float* ws_stats,
                 float output_scale, void* o, bool o_is_f32, float* lse, void* stream,
                 const DeviceArgs* dev = nullptr, const MergeEpilogue* epi = nullptr);
// Split partials from their sub-ranges' partial states (dev.subs > 1): reads sub_o /
// sub_stats ([split][sub][row]), writes o / stats ([split][row]).
int launch_fold(const mla_decode_plan_s& plan, const float* sub_o, const float* sub_stats,
                float* o, float* stats, void* stream, const DeviceArgs* dev = nullptr);
// Splits that fill the chip once for row blocks of `tiles` (XCD-aware; plan.cpp).
int64_t split_budget(int32_t num_cus, int32_t tiles);
int launch_device_plan(const mla_decode_plan_s& plan, const int32_t* kv_lens, PlanDev* out,
                       void* stream);

}  // namespace mla
