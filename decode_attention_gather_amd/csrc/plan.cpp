// Host split planner for split-KV MLA decode.
//
// Prior art: the per-request split plan of TensorRT-LLM issue #20510 "CuTe DSL FP8 MLA
// decode slower after #19338" (Repro 2: block_split_kvs from the planner, a per-request
// cap raised to 128 so that a single request can occupy the whole GPU; follow-up comment: the plan
// clamped to [1, split_kv], and a minimum split length of one tile rather than four at
// short KV) and the grid rule of its Repro 1 (uniform split_kv so that B * split_kv is
// about one wave). Here a wave is one workgroup per CU on a 256-CU MI355X, and a work
// item is one (split, 16-row tile); the merge-width rule follows PR #20380 "trtllm-gen
// FMHA: split the KV partials of a row across thread groups in fmhaReductionKernel"
// (Description: an upper bound halved until the launch fits a 2-per-CU budget).
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "mla_internal.h"

namespace mla {

int query_num_cus(int32_t* out);  // abi.hip (HIP runtime)

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Splits that fill the chip once. Workgroup i runs on XCD i mod 8 and the row blocks of
// one split are issued to one XCD, so a wave holds floor(CUs per XCD / row blocks)
// splits per XCD; a plan above that leaves some XCD with more workgroups than CUs and
// the whole launch waits for a second round there.
int64_t split_budget(int32_t num_cus, int32_t tiles) {
  const int64_t per_xcd = (int64_t)(num_cus / kXcds) / tiles;
  if (per_xcd >= 1) return per_xcd * kXcds;
  return std::max<int64_t>(1, num_cus / tiles);
}

namespace {

// Splits wanted per request before clamping.
void want_splits(const std::vector<int64_t>& pages, int32_t split_kv, int32_t max_split,
                 int32_t tiles, int32_t num_cus, std::vector<int64_t>& want) {
  const size_t B = pages.size();
  want.assign(B, 1);
  if (split_kv > 0) {
    for (size_t b = 0; b < B; ++b) want[b] = std::min<int64_t>(split_kv, max_split);
    return;
  }
  // Proportional plan: S_b = ceil(pages_b / C) with C the smallest split length (pages)
  // for which sum_b clamp(ceil(pages_b / C), 1, cap) fits the one-wave split budget. The
  // splits follow the lengths, and the rounding keeps the longest split, which the whole
  // launch waits for, as short as the budget allows (flooring each request's share of
  // the budget instead can leave one request's splits nearly twice the mean).
  const int64_t budget = split_budget(num_cus, tiles);
  int64_t total = 0, max_p = 1;
  for (int64_t p : pages) {
    total += p;
    max_p = std::max(max_p, p);
  }
  auto count = [&](int64_t C) {
    int64_t n = 0;
    for (int64_t p : pages) n += std::min<int64_t>(std::max<int64_t>(ceil_div(p, C), 1), max_split);
    return n;
  };
  // C = max_p gives one split per request; with budget > B, C = ceil(total / (budget - B))
  // fits as well, since sum_b ceil(p_b / C) < total / C + B
  const int64_t Bn = (int64_t)B;
  int64_t lo = 1, hi = max_p;
  if (budget > Bn) hi = std::min(hi, ceil_div(total, budget - Bn));
  else lo = hi;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (count(mid) <= budget) hi = mid; else lo = mid + 1;
  }
  for (size_t b = 0; b < B; ++b)
    want[b] = std::min<int64_t>(std::max<int64_t>(ceil_div(pages[b], lo), 1), max_split);
}

// Row blocks of 16-row MFMA tiles. Up to 32 rows: one block of 1 or 2 tiles (narrow
// kernel). More rows: blocks of 4 or 6 tiles (wide kernel), as few as 96-row blocks
// allow, so that one staged page feeds as many rows as the workgroup holds. Both cache
// types follow the rule (each has a narrow and a wide kernel).
void row_blocks(int32_t rows, int32_t* tiles, int32_t* nt) {
  const int32_t tiles16 = (int32_t)ceil_div(rows, kTileRows);
  if (tiles16 <= kMaxTilesPerBlock) {
    *tiles = 1;
    *nt = tiles16;
  } else {
    const int32_t blocks = (int32_t)ceil_div(tiles16, kWideMaxTiles);
    *nt = ceil_div(tiles16, blocks) <= 4 ? 4 : kWideMaxTiles;
    *tiles = (int32_t)ceil_div(tiles16, *nt);
  }
}

// Merge width: wavefront groups per row, a power of two <= min(16, max splits), halved
// while the waves that fold partials, sum over requests of rows x min(groups, S_b),
// exceed what the CUs hold at once: two 16-wave workgroups, 32 waves, per CU (the
// pages' rule halves the width until the launch fits its two-per-SM budget). Groups
// beyond a row's split count have nothing to fold and end at once, so a short request
// beside a long one (a skewed batch) does not hold the long one's rows to a narrow merge.
int32_t merge_groups_for(const std::vector<int64_t>& splits, int64_t rows, int32_t num_cus) {
  int64_t max_s = 0;
  for (int64_t sb : splits) max_s = std::max(max_s, sb);
  int32_t g = 1;
  while (g * 2 <= 16 && g * 2 <= max_s) g *= 2;
  auto waves = [&](int32_t gg) {
    int64_t w = 0;
    for (int64_t sb : splits) w += rows * std::min<int64_t>(gg, sb);
    return w;
  };
  while (g > 1 && waves(g) > (int64_t)kMergeWavesPerCu * num_cus) g /= 2;
  return g;
}

// Merge slices: a row's 512 output dims may be split over W = 8 workgroups. Measured
// on the merge kernel: more workgroups help only when very few rows hold many splits
// (one long request at q = 1: 12 rows x 256 splits, 11.1 -> 8.0 us), where each
// wavefront would otherwise walk its partials in several dependent rounds; elsewhere
// the extra waves cost more than they give (192 rows x 16 splits: 6.2 -> 7.1 us; a
// skewed batch: 13.4 -> 50 us). So W = 8 when the rows of the requests with the most
// splits (S_b at least half the largest) number at most num_cus / 16 and those requests
// have more than 16 x 8 splits (several rounds per wavefront even at 16 groups); else
// 1. The slices do not change
// any sum's order (each dim is still folded by one lane), and the merge width above
// ignores them, so host and graph plans of the same lengths give the same bits.
int32_t merge_slices_for(const std::vector<int64_t>& splits, int64_t rows, int32_t num_cus) {
  int64_t max_s = 0, heavy = 0;
  for (int64_t sb : splits) max_s = std::max(max_s, sb);
  for (int64_t sb : splits)
    if (2 * sb >= max_s) heavy += rows;
  return (heavy * 16 <= num_cus && max_s > 16 * 8) ? kMaxMergeSlices : 1;
}

}  // namespace

int build_plan(const int32_t* kv_lens_host, int32_t batch, int32_t q_len, int32_t num_heads,
               int32_t split_kv, int32_t max_split_kv, int32_t num_cus, int32_t kv_dtype,
               mla_decode_plan_s** out) {
  if (out == nullptr) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (kv_lens_host == nullptr || batch < 1 || q_len < 1 || num_heads < 1 || split_kv < 0 ||
      max_split_kv < 1 || num_cus < 0 || (kv_dtype != MLA_KV_E4M3 && kv_dtype != MLA_KV_BF16))
    return MLA_ERR_INVALID_ARG;
  if (batch > kMaxBatch || max_split_kv > MLA_MAX_SPLIT_KV ||
      (int64_t)q_len * num_heads > MLA_MAX_ROWS_PER_REQUEST)
    return MLA_ERR_UNSUPPORTED_SHAPE;
  for (int32_t b = 0; b < batch; ++b)
    if (kv_lens_host[b] < q_len) return MLA_ERR_INVALID_ARG;
  if (num_cus == 0) {
    int rc = query_num_cus(&num_cus);
    if (rc != MLA_OK) return rc;
  }

  const int32_t rows = q_len * num_heads;
  int32_t tiles, nt;
  row_blocks(rows, &tiles, &nt);
  std::vector<int64_t> pages(batch), want;
  for (int32_t b = 0; b < batch; ++b) pages[b] = ceil_div(kv_lens_host[b], kPage);
  want_splits(pages, split_kv, max_split_kv, tiles, num_cus, want);

  auto* plan = new (std::nothrow) mla_decode_plan_s();
  if (plan == nullptr) return MLA_ERR_NOMEM;
  plan->kv_lens = (int32_t*)std::malloc(sizeof(int32_t) * batch);
  if (plan->kv_lens == nullptr) {
    delete plan;
    return MLA_ERR_NOMEM;
  }
  std::memcpy(plan->kv_lens, kv_lens_host, sizeof(int32_t) * batch);
  plan->kv_dtype = kv_dtype;

  PlanDev& d = plan->dev;
  std::memset(&d, 0, sizeof(d));
  d.batch = batch;
  d.q_len = q_len;
  d.heads = num_heads;
  d.rows = rows;
  d.tiles = tiles;
  d.nt = nt;

  int64_t total = 0, max_s = 0;
  std::vector<int64_t> chunk_of(batch), split_of(batch);
  for (int32_t b = 0; b < batch; ++b) {
    // whole pages per split, no empty split, split length within uint16 pages
    int64_t s = std::max<int64_t>(1, std::min<int64_t>(want[b], pages[b]));
    s = std::max<int64_t>(s, ceil_div(pages[b], kMaxChunkPages));
    int64_t chunk = ceil_div(pages[b], s);
    s = ceil_div(pages[b], chunk);
    d.splits[b] = (uint16_t)s;
    d.kv_len[b] = (uint32_t)kv_lens_host[b];
    d.part_base[b] = (uint32_t)total;
    chunk_of[b] = chunk;
    split_of[b] = s;
    total += s;
    max_s = std::max(max_s, s);
  }
  if (total * tiles > INT32_MAX / 2 || total >= (1 << 23)) {
    mla_decode_plan_destroy(plan);
    return MLA_ERR_UNSUPPORTED_SHAPE;
  }
  d.total_parts = (int32_t)total;

  // Cooperative splits. A grid of at most half as many work items as CUs (a fixed
  // split_kv over few requests) runs each split on `subs` workgroups, every one over a
  // run of whole steps of the split's pages, and a fold kernel combines their partial
  // states into the split's partial: the idle CUs then share the split's key range,
  // where otherwise each busy CU walks its whole split one step at a time. A run keeps
  // at least kMinSubSteps steps of the longest split. The partials the pass writes are
  // still one per (split, row).
  int64_t max_steps = 0;
  for (int32_t b = 0; b < batch; ++b) max_steps = std::max(max_steps, ceil_div(chunk_of[b], 2));
  auto subs_for = [&](int64_t items) {
    const int64_t by_cus = num_cus / items;
    const int64_t by_len = max_steps / kMinSubSteps;
    return (int32_t)std::max<int64_t>(1, std::min<int64_t>({by_cus, by_len, kMaxSubs}));
  };
  // A split plan that leaves CUs idle with 96-row blocks and cannot share its splits
  // takes blocks of 64 rows instead when the larger grid still fits one wave of the
  // chip: a work item then costs about two thirds as much, and the extra reads of each
  // page come from idle CUs' share of HBM. Shared splits are the better use of idle CUs
  // where they apply (each page still crosses HBM once per 96 rows). A row's arithmetic
  // does not depend on its block.
  if (nt == kWideMaxTiles && subs_for(total * tiles) < 2) {
    const int32_t tiles4 = (int32_t)ceil_div(ceil_div(rows, kTileRows), 4);
    if (total <= split_budget(num_cus, tiles4)) {
      d.nt = 4;
      d.tiles = tiles = tiles4;
    }
  }
  const int32_t subs = subs_for(total * tiles);
  d.subs = subs;

  // Longest request first, so the longest work items start in the first wave.
  std::vector<int32_t> order(batch);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return chunk_of[a] > chunk_of[b]; });
  uint32_t run = 0;
  for (int32_t e = 0; e < batch; ++e) {
    run += d.splits[order[e]];
    d.sorted[e] = (run << 8) | (uint32_t)order[e];
  }

  plan->merge_slices = merge_slices_for(split_of, rows, num_cus);
  plan->merge_groups = merge_groups_for(split_of, rows, num_cus);
  d.groups = plan->merge_groups;
  plan->max_splits = (int32_t)max_s;
  plan->num_cus = num_cus;
  plan->ws_o_bytes = align256((size_t)total * rows * kDV * sizeof(float));
  plan->ws_stats_bytes = align256((size_t)total * rows * kStatStride * sizeof(float));
  if (subs > 1) {
    plan->ws_sub_o_bytes = align256((size_t)total * subs * rows * kDV * sizeof(float));
    plan->ws_sub_stats_bytes = align256((size_t)total * subs * rows * kStatStride * sizeof(float));
  }
  *out = plan;
  return MLA_OK;
}

// Graph plan: shapes and upper bounds only; the device planner fills in the splits on
// every call. Capacity (work items the launches are sized for):
//   uniform split_kv:  B * max(min(split_kv, cap), ceil(max_pages / 65535))
//   proportional:      min(B * cap, 2 B + split budget)   (+ B * ceil(max_pages /
//                      65535) beyond 2^21 tokens), since sum_b floor(x_b) <= sum_b x_b and
//                      the clamps to >= 1 add at most one split per request.
int build_graph_plan(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_kv_len,
                     int32_t split_kv, int32_t max_split_kv, int32_t num_cus, int32_t kv_dtype,
                     mla_decode_plan_s** out) {
  if (out == nullptr) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (batch < 1 || q_len < 1 || num_heads < 1 || max_kv_len < 1 || split_kv < 0 ||
      max_split_kv < 1 || num_cus < 0 || (kv_dtype != MLA_KV_E4M3 && kv_dtype != MLA_KV_BF16))
    return MLA_ERR_INVALID_ARG;
  if (batch > kMaxBatch || max_split_kv > MLA_MAX_SPLIT_KV ||
      (int64_t)q_len * num_heads > MLA_MAX_ROWS_PER_REQUEST)
    return MLA_ERR_UNSUPPORTED_SHAPE;
  if (num_cus == 0) {
    int rc = query_num_cus(&num_cus);
    if (rc != MLA_OK) return rc;
  }
  const int32_t rows = q_len * num_heads;
  int32_t tiles, nt;
  row_blocks(rows, &tiles, &nt);
  const int64_t max_pages = ceil_div(max_kv_len, kPage);
  const int64_t long_split = ceil_div(max_pages, kMaxChunkPages);  // forced splits per request
  int64_t per_req, cap;
  if (split_kv > 0) {
    per_req = std::max<int64_t>(std::min<int64_t>(split_kv, max_split_kv), long_split);
    cap = (int64_t)batch * per_req;
  } else {
    per_req = std::max<int64_t>(max_split_kv, long_split);
    cap = std::min<int64_t>((int64_t)batch * max_split_kv, 2LL * batch + split_budget(num_cus, tiles));
    if (long_split > 1) cap += (int64_t)batch * long_split;
  }
  per_req = std::min<int64_t>(per_req, max_pages);
  cap = std::min<int64_t>(cap, (int64_t)batch * max_pages);
  if (cap * tiles > INT32_MAX / 2 || cap >= (1 << 23)) return MLA_ERR_UNSUPPORTED_SHAPE;

  auto* plan = new (std::nothrow) mla_decode_plan_s();
  if (plan == nullptr) return MLA_ERR_NOMEM;
  PlanDev& d = plan->dev;
  std::memset(&d, 0, sizeof(d));
  d.batch = batch;
  d.q_len = q_len;
  d.heads = num_heads;
  d.rows = rows;
  d.tiles = tiles;
  d.nt = nt;
  d.total_parts = (int32_t)cap;
  // Shared splits as in host plans, decided here from the capacity and the length bound
  // (uniform split_kv only: the proportional planner fills the chip); the device planner
  // copies the count into every device plan.
  d.subs = 1;
  if (split_kv > 0) {
    const int64_t longest = ceil_div(max_pages, std::min<int64_t>(per_req, max_pages));
    const int64_t by_cus = num_cus / (cap * tiles);
    const int64_t by_len = ceil_div(longest, 2) / kMinSubSteps;
    d.subs = (int32_t)std::max<int64_t>(1, std::min<int64_t>({by_cus, by_len, kMaxSubs}));
  }
  plan->device_lengths = 1;
  plan->kv_dtype = kv_dtype;
  plan->max_kv_len = max_kv_len;
  plan->split_kv = split_kv;
  plan->max_split_kv = max_split_kv;
  plan->kv_lens = nullptr;
  // merge slices as for a batch of equal requests at the largest split count
  plan->merge_slices = merge_slices_for(std::vector<int64_t>(batch, per_req), rows, num_cus);
  // launch width: at most min(16, largest split count), halved while the launch would
  // start more than 64 waves per CU (B rows G); the device planner applies the host rule
  // to the actual splits and picks <= this, so graph and host plans of the same lengths
  // merge alike whenever the host's width fits under it. A launch at the unhalved width
  // starts 16 waves per row even where one folds everything (6144 rows: 39 us of merge).
  {
    int32_t g = 1;
    while (g * 2 <= 16 && g * 2 <= per_req) g *= 2;
    while (g > 1 && (int64_t)batch * rows * g > 2LL * kMergeWavesPerCu * num_cus) g /= 2;
    plan->merge_groups = g;
  }
  d.groups = plan->merge_groups;
  plan->max_splits = (int32_t)per_req;
  plan->num_cus = num_cus;
  plan->ws_plan_bytes = align256(sizeof(PlanDev));
  plan->ws_o_bytes = align256((size_t)cap * rows * kDV * sizeof(float));
  plan->ws_stats_bytes = align256((size_t)cap * rows * kStatStride * sizeof(float));
  if (d.subs > 1) {
    plan->ws_sub_o_bytes = align256((size_t)cap * d.subs * rows * kDV * sizeof(float));
    plan->ws_sub_stats_bytes =
        align256((size_t)cap * d.subs * rows * kStatStride * sizeof(float));
  }
  *out = plan;
  return MLA_OK;
}

}  // namespace mla

extern "C" {

int mla_decode_plan_graph(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_kv_len,
                          int32_t split_kv, int32_t max_split_kv, int32_t num_cus,
                          mla_decode_plan_t** out) {
  return mla::build_graph_plan(batch, q_len, num_heads, max_kv_len, split_kv, max_split_kv,
                               num_cus, MLA_KV_E4M3, out);
}

int mla_decode_plan_graph_ex(int32_t batch, int32_t q_len, int32_t num_heads,
                             int32_t max_kv_len, int32_t split_kv, int32_t max_split_kv,
                             int32_t num_cus, int32_t kv_dtype, mla_decode_plan_t** out) {
  return mla::build_graph_plan(batch, q_len, num_heads, max_kv_len, split_kv, max_split_kv,
                               num_cus, kv_dtype, out);
}

int mla_decode_plan(const int32_t* kv_lens_host, int32_t batch, int32_t q_len,
                    int32_t num_heads, int32_t split_kv, int32_t max_split_kv,
                    int32_t num_cus, mla_decode_plan_t** out) {
  return mla::build_plan(kv_lens_host, batch, q_len, num_heads, split_kv, max_split_kv,
                         num_cus, MLA_KV_E4M3, out);
}

int mla_decode_plan_ex(const int32_t* kv_lens_host, int32_t batch, int32_t q_len,
                       int32_t num_heads, int32_t split_kv, int32_t max_split_kv,
                       int32_t num_cus, int32_t kv_dtype, mla_decode_plan_t** out) {
  return mla::build_plan(kv_lens_host, batch, q_len, num_heads, split_kv, max_split_kv,
                         num_cus, kv_dtype, out);
}

int mla_decode_plan_with_merge_bound(const mla_decode_plan_t* plan, int32_t max_groups,
                                     mla_decode_plan_t** out) {
  if (out == nullptr) return MLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (plan == nullptr || max_groups < 1 || max_groups > 16 || (max_groups & (max_groups - 1)))
    return MLA_ERR_INVALID_ARG;
  auto* copy = new (std::nothrow) mla_decode_plan_s(*plan);
  if (copy == nullptr) return MLA_ERR_NOMEM;
  copy->kv_lens = nullptr;
  if (plan->kv_lens != nullptr) {
    copy->kv_lens = (int32_t*)std::malloc(sizeof(int32_t) * plan->dev.batch);
    if (copy->kv_lens == nullptr) {
      delete copy;
      return MLA_ERR_NOMEM;
    }
    std::memcpy(copy->kv_lens, plan->kv_lens, sizeof(int32_t) * plan->dev.batch);
  }
  // The planner's width is the largest power of two <= min(16, max S_b), halved while the
  // launch exceeds its budget; the budget test is monotone in the width, so applying the
  // bound first and then halving gives min(bound, planner's width). Graph plans: this is
  // the launch width, which also caps the device planner's choice.
  copy->merge_groups = std::min(plan->merge_groups, max_groups);
  copy->dev.groups = std::min<int32_t>(plan->dev.groups, copy->merge_groups);
  *out = copy;
  return MLA_OK;
}

void mla_decode_plan_destroy(mla_decode_plan_t* plan) {
  if (plan == nullptr) return;
  std::free(plan->kv_lens);
  delete plan;
}

size_t mla_decode_workspace_size(const mla_decode_plan_t* plan) {
  if (plan == nullptr) return 0;
  return mla::workspace_bytes_of(*plan);
}

int mla_decode_plan_get_info(const mla_decode_plan_t* plan, mla_decode_plan_info_t* info,
                             int32_t* splits, int32_t* chunk_tokens) {
  if (plan == nullptr || info == nullptr) return MLA_ERR_INVALID_ARG;
  const mla::PlanDev& d = plan->dev;
  info->batch = d.batch;
  info->q_len = d.q_len;
  info->num_heads = d.heads;
  info->rows_per_request = d.rows;
  info->row_tiles = d.tiles;
  info->total_splits = d.total_parts;
  info->work_items = d.total_parts * d.tiles;
  info->split_workgroups = d.subs;
  info->merge_groups = plan->merge_groups;
  info->merge_slices = plan->merge_slices;
  info->max_splits = plan->max_splits;
  for (int32_t b = 0; b < d.batch; ++b) {  // graph plans: decided on the device, 0 here
    if (splits) splits[b] = plan->device_lengths ? 0 : d.splits[b];
    if (chunk_tokens)
      chunk_tokens[b] = plan->device_lengths ? 0 : mla::chunk_pages_of(d, b) * mla::kPage;
  }
  return MLA_OK;
}

}  // extern "C"
