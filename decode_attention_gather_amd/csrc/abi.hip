// C-ABI entry points of libmla_decode.so: argument checks on the host, then the two
// kernel launches on the caller's stream. Nothing here allocates device memory or
// synchronises; every check runs before the first launch, so a rejected call enqueues
// nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mla_internal.h"

namespace mla {

int query_num_cus(int32_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return MLA_ERR_HIP_BASE - (int)e;
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return MLA_ERR_HIP_BASE - (int)e;
  if (n <= 0) return MLA_ERR_HIP_BASE - (int)hipErrorInvalidDevice;
  *out = n;
  return MLA_OK;
}

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_workspace(const mla_decode_plan_s* plan, const void* ws, size_t bytes) {
  if (ws == nullptr || !aligned(ws, 256)) return MLA_ERR_WORKSPACE;
  if (bytes < workspace_bytes_of(*plan)) return MLA_ERR_WORKSPACE;
  return MLA_OK;
}

int check_partial(const mla_decode_plan_s* plan, const void* q, const void* kv,
                  const int32_t* bt, int64_t bt_stride, const int32_t* kv_lens,
                  float softmax_scale, const void* ws, size_t ws_bytes) {
  if (plan == nullptr || q == nullptr || kv == nullptr || bt == nullptr || kv_lens == nullptr)
    return MLA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(bt, 4) || !aligned(kv_lens, 4))
    return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale) || __builtin_isinf(softmax_scale))
    return MLA_ERR_INVALID_ARG;
  // every request's pages must fit its block-table row
  int64_t max_pages = 0;
  if (plan->device_lengths) {
    max_pages = ((int64_t)plan->max_kv_len + kPage - 1) / kPage;
  } else {
    for (int32_t b = 0; b < plan->dev.batch; ++b) {
      const int64_t p = ((int64_t)plan->kv_lens[b] + kPage - 1) / kPage;
      if (p > max_pages) max_pages = p;
    }
  }
  if (bt_stride < max_pages) return MLA_ERR_INVALID_ARG;
  return check_workspace(plan, ws, ws_bytes);
}

int check_merge(const mla_decode_plan_s* plan, const void* ws, size_t ws_bytes,
                float output_scale, const void* o, const float* lse) {
  if (plan == nullptr || o == nullptr) return MLA_ERR_INVALID_ARG;
  if (!aligned(o, 4) || (lse != nullptr && !aligned(lse, 4))) return MLA_ERR_INVALID_ARG;
  if (!(output_scale == output_scale) || __builtin_isinf(output_scale))
    return MLA_ERR_INVALID_ARG;
  return check_workspace(plan, ws, ws_bytes);
}

// Merge outputs with the epilogue options: o (BF16) may be null when the MXFP8 pair is
// given; the pair is both-or-neither; the MXFP8 store writes 16 B of BF16 and 8 B of
// codes per lane, hence the alignments.
int check_epilogue(const mla_decode_plan_s* plan, const void* ws, size_t ws_bytes,
                   float output_scale, const void* o, const float* lse, const float* sinks,
                   const void* o_fp8, const void* o_fp8_scales) {
  if ((o_fp8 == nullptr) != (o_fp8_scales == nullptr)) return MLA_ERR_INVALID_ARG;
  if (sinks != nullptr && !aligned(sinks, 4)) return MLA_ERR_INVALID_ARG;
  if (o_fp8 != nullptr) {
    if (!aligned(o_fp8, 8) || (o != nullptr && !aligned(o, 16))) return MLA_ERR_INVALID_ARG;
    if (o == nullptr) o = o_fp8;  // only the BF16 pointer may be absent
  }
  return check_merge(plan, ws, ws_bytes, output_scale, o, lse);
}

int hip_status(int e) { return e == (int)hipSuccess ? MLA_OK : MLA_ERR_HIP_BASE - e; }

// Partials scratch of mla_decode_noalloc: one array per GPU, loaded with the library's
// code object and held until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the address hipGetSymbolAddress returns for
// the current device, looked up once per device and kept in scratch_ptr.
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return MLA_ERR_HIP_BASE - (int)e;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED_SHAPE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return MLA_ERR_HIP_BASE - (int)e;
    if (p == nullptr) return MLA_ERR_HIP_BASE - (int)hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MLA_OK;
}

float* ws_o_of(const mla_decode_plan_s* plan, const void* ws) {
  return (float*)((uint8_t*)ws + plan->ws_plan_bytes);
}
float* ws_stats_of(const mla_decode_plan_s* plan, const void* ws) {
  return (float*)((uint8_t*)ws + plan->ws_plan_bytes + plan->ws_o_bytes);
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

int mla_decode_partial(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                       const int32_t* block_table, int64_t bt_stride,
                       const int32_t* kv_lens, float softmax_scale, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, softmax_scale,
                         workspace, workspace_bytes);
  if (rc != MLA_OK) return rc;
  return hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache,
                                   block_table, bt_stride, kv_lens, softmax_scale,
                                   ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                   stream));
}

int mla_decode_merge(const mla_decode_plan_t* plan, const void* workspace,
                     size_t workspace_bytes, float output_scale, void* o, float* lse,
                     void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  int rc = check_merge(plan, workspace, workspace_bytes, output_scale, o, lse);
  if (rc != MLA_OK) return rc;
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 output_scale, o, false, lse, stream));
}

int mla_decode_merge_f32(const mla_decode_plan_t* plan, const void* workspace,
                         size_t workspace_bytes, float output_scale, float* o, float* lse,
                         void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  int rc = check_merge(plan, workspace, workspace_bytes, output_scale, o, lse);
  if (rc != MLA_OK) return rc;
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 output_scale, o, true, lse, stream));
}

int mla_decode(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
               const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
               float softmax_scale, float output_scale, void* workspace,
               size_t workspace_bytes, void* o, float* lse, void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, softmax_scale,
                         workspace, workspace_bytes);
  if (rc != MLA_OK) return rc;
  rc = check_merge(plan, workspace, workspace_bytes, output_scale, o, lse);
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache,
                                 block_table, bt_stride, kv_lens, softmax_scale,
                                 ws_o_of(plan, workspace), ws_stats_of(plan, workspace), stream));
  if (rc != MLA_OK) return rc;
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 output_scale, o, false, lse, stream));
}

int mla_decode_noalloc(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                       const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                       float softmax_scale, float output_scale, void* o, float* lse,
                       void* stream) {
  if (plan == nullptr || plan->device_lengths) return MLA_ERR_INVALID_ARG;
  const size_t need = workspace_bytes_of(*plan);
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  int rc = scratch_of_current_device(&ws);
  if (rc != MLA_OK) return rc;
  // the same checks and kernels as mla_decode, with the scratch as the workspace; every
  // partial the merge reads is written by the partial pass of the same call, so nothing
  // in the scratch needs clearing
  rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, softmax_scale, ws,
                     (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  if (rc != MLA_OK) return rc;
  rc = check_merge(plan, ws, (size_t)MLA_NOALLOC_SCRATCH_BYTES, output_scale, o, lse);
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache,
                                 block_table, bt_stride, kv_lens, softmax_scale,
                                 ws_o_of(plan, ws), ws_stats_of(plan, ws), stream));
  if (rc != MLA_OK) return rc;
  return hip_status(launch_merge(*plan, ws_o_of(plan, ws), ws_stats_of(plan, ws), output_scale,
                                 o, false, lse, stream));
}

int mla_decode_varq(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                    const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                    const int32_t* q_lens, float softmax_scale, float output_scale,
                    void* workspace, size_t workspace_bytes, void* o, float* lse,
                    void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  if (q_lens == nullptr || !aligned(q_lens, 4)) return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, softmax_scale,
                         workspace, workspace_bytes);
  if (rc != MLA_OK) return rc;
  rc = check_merge(plan, workspace, workspace_bytes, output_scale, o, lse);
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache,
                                 block_table, bt_stride, kv_lens, softmax_scale,
                                 ws_o_of(plan, workspace), ws_stats_of(plan, workspace), stream,
                                 nullptr, q_lens));
  if (rc != MLA_OK) return rc;
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 output_scale, o, false, lse, stream));
}

int mla_decode_graph(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                     const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                     const int32_t* q_lens, const float* softmax_scale, const float* output_scale,
                     void* workspace, size_t workspace_bytes, void* o, float* lse,
                     void* stream) {
  if (plan == nullptr || !plan->device_lengths) return MLA_ERR_INVALID_ARG;
  if (q_lens != nullptr && !aligned(q_lens, 4)) return MLA_ERR_INVALID_ARG;
  if (softmax_scale == nullptr || output_scale == nullptr || !aligned(softmax_scale, 4) ||
      !aligned(output_scale, 4))
    return MLA_ERR_INVALID_ARG;
  // the scale values live on the device: a finite placeholder passes the host check
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, 1.f, workspace,
                         workspace_bytes);
  if (rc != MLA_OK) return rc;
  rc = check_merge(plan, workspace, workspace_bytes, 1.f, o, lse);
  if (rc != MLA_OK) return rc;
  PlanDev* pdev = (PlanDev*)workspace;
  const DeviceArgs dev{pdev, softmax_scale, output_scale};
  rc = hip_status(launch_device_plan(*plan, kv_lens, pdev, stream));
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache, block_table,
                                 bt_stride, kv_lens, 1.f, ws_o_of(plan, workspace),
                                 ws_stats_of(plan, workspace), stream, &dev, q_lens));
  if (rc != MLA_OK) return rc;
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace), 1.f,
                                 o, false, lse, stream, &dev));
}

int mla_decode_merge_ex(const mla_decode_plan_t* plan, const void* workspace,
                        size_t workspace_bytes, float output_scale, const float* sinks, void* o,
                        float* lse, void* o_fp8, void* o_fp8_scales, void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  int rc = check_epilogue(plan, workspace, workspace_bytes, output_scale, o, lse, sinks, o_fp8,
                          o_fp8_scales);
  if (rc != MLA_OK) return rc;
  const MergeEpilogue ep{sinks, (uint8_t*)o_fp8, (uint8_t*)o_fp8_scales};
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 output_scale, o, false, lse, stream, nullptr, &ep));
}

int mla_decode_ex(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                  const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                  const int32_t* q_lens, float softmax_scale, float output_scale,
                  const float* sinks, void* workspace, size_t workspace_bytes, void* o,
                  float* lse, void* o_fp8, void* o_fp8_scales, void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  if (q_lens != nullptr && !aligned(q_lens, 4)) return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, softmax_scale,
                         workspace, workspace_bytes);
  if (rc != MLA_OK) return rc;
  rc = check_epilogue(plan, workspace, workspace_bytes, output_scale, o, lse, sinks, o_fp8,
                      o_fp8_scales);
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache,
                                 block_table, bt_stride, kv_lens, softmax_scale,
                                 ws_o_of(plan, workspace), ws_stats_of(plan, workspace), stream,
                                 nullptr, q_lens));
  if (rc != MLA_OK) return rc;
  const MergeEpilogue ep{sinks, (uint8_t*)o_fp8, (uint8_t*)o_fp8_scales};
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 output_scale, o, false, lse, stream, nullptr, &ep));
}

int mla_decode_graph_ex(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                        const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                        const int32_t* q_lens, const float* softmax_scale,
                        const float* output_scale, const float* sinks, void* workspace,
                        size_t workspace_bytes, void* o, float* lse, void* o_fp8,
                        void* o_fp8_scales, void* stream) {
  if (plan == nullptr || !plan->device_lengths) return MLA_ERR_INVALID_ARG;
  if (q_lens != nullptr && !aligned(q_lens, 4)) return MLA_ERR_INVALID_ARG;
  if (softmax_scale == nullptr || output_scale == nullptr || !aligned(softmax_scale, 4) ||
      !aligned(output_scale, 4))
    return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, 1.f, workspace,
                         workspace_bytes);
  if (rc != MLA_OK) return rc;
  rc = check_epilogue(plan, workspace, workspace_bytes, 1.f, o, lse, sinks, o_fp8, o_fp8_scales);
  if (rc != MLA_OK) return rc;
  PlanDev* pdev = (PlanDev*)workspace;
  const DeviceArgs dev{pdev, softmax_scale, output_scale};
  rc = hip_status(launch_device_plan(*plan, kv_lens, pdev, stream));
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache, block_table,
                                 bt_stride, kv_lens, 1.f, ws_o_of(plan, workspace),
                                 ws_stats_of(plan, workspace), stream, &dev, q_lens));
  if (rc != MLA_OK) return rc;
  const MergeEpilogue ep{sinks, (uint8_t*)o_fp8, (uint8_t*)o_fp8_scales};
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 1.f, o, false, lse, stream, &dev, &ep));
}

int mla_decode_partial_ex(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                          const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                          const int32_t* q_lens, const int32_t* kv_bounds, float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  if ((q_lens != nullptr && !aligned(q_lens, 4)) || (kv_bounds != nullptr && !aligned(kv_bounds, 4)))
    return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, softmax_scale,
                         workspace, workspace_bytes);
  if (rc != MLA_OK) return rc;
  return hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache,
                                   block_table, bt_stride, kv_lens, softmax_scale,
                                   ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                   stream, nullptr, q_lens, kv_bounds));
}

int mla_decode_bounded(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                       const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                       const int32_t* q_lens, const int32_t* kv_bounds, float softmax_scale,
                       float output_scale, const float* sinks, void* workspace,
                       size_t workspace_bytes, void* o, float* lse, void* o_fp8,
                       void* o_fp8_scales, void* stream) {
  if (plan != nullptr && plan->device_lengths) return MLA_ERR_INVALID_ARG;
  if (kv_bounds == nullptr || !aligned(kv_bounds, 4)) return MLA_ERR_INVALID_ARG;
  if (q_lens != nullptr && !aligned(q_lens, 4)) return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, softmax_scale,
                         workspace, workspace_bytes);
  if (rc != MLA_OK) return rc;
  rc = check_epilogue(plan, workspace, workspace_bytes, output_scale, o, lse, sinks, o_fp8,
                      o_fp8_scales);
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache,
                                 block_table, bt_stride, kv_lens, softmax_scale,
                                 ws_o_of(plan, workspace), ws_stats_of(plan, workspace), stream,
                                 nullptr, q_lens, kv_bounds));
  if (rc != MLA_OK) return rc;
  const MergeEpilogue ep{sinks, (uint8_t*)o_fp8, (uint8_t*)o_fp8_scales};
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 output_scale, o, false, lse, stream, nullptr, &ep));
}

int mla_decode_graph_bounded(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                             const int32_t* block_table, int64_t bt_stride,
                             const int32_t* kv_lens, const int32_t* q_lens,
                             const int32_t* kv_bounds, const float* softmax_scale,
                             const float* output_scale, const float* sinks, void* workspace,
                             size_t workspace_bytes, void* o, float* lse, void* o_fp8,
                             void* o_fp8_scales, void* stream) {
  if (plan == nullptr || !plan->device_lengths) return MLA_ERR_INVALID_ARG;
  if (kv_bounds == nullptr || !aligned(kv_bounds, 4)) return MLA_ERR_INVALID_ARG;
  if (q_lens != nullptr && !aligned(q_lens, 4)) return MLA_ERR_INVALID_ARG;
  if (softmax_scale == nullptr || output_scale == nullptr || !aligned(softmax_scale, 4) ||
      !aligned(output_scale, 4))
    return MLA_ERR_INVALID_ARG;
  int rc = check_partial(plan, q, kv_cache, block_table, bt_stride, kv_lens, 1.f, workspace,
                         workspace_bytes);
  if (rc != MLA_OK) return rc;
  rc = check_epilogue(plan, workspace, workspace_bytes, 1.f, o, lse, sinks, o_fp8, o_fp8_scales);
  if (rc != MLA_OK) return rc;
  PlanDev* pdev = (PlanDev*)workspace;
  const DeviceArgs dev{pdev, softmax_scale, output_scale};
  rc = hip_status(launch_device_plan(*plan, kv_lens, pdev, stream));
  if (rc != MLA_OK) return rc;
  rc = hip_status(launch_partial(*plan, (const uint8_t*)q, (const uint8_t*)kv_cache, block_table,
                                 bt_stride, kv_lens, 1.f, ws_o_of(plan, workspace),
                                 ws_stats_of(plan, workspace), stream, &dev, q_lens, kv_bounds));
  if (rc != MLA_OK) return rc;
  const MergeEpilogue ep{sinks, (uint8_t*)o_fp8, (uint8_t*)o_fp8_scales};
  return hip_status(launch_merge(*plan, ws_o_of(plan, workspace), ws_stats_of(plan, workspace),
                                 1.f, o, false, lse, stream, &dev, &ep));
}

const char* mla_decode_strerror(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (batch, rows per request or split cap)";
    case MLA_ERR_WORKSPACE: return "workspace missing, misaligned (256 B) or smaller than mla_decode_workspace_size()";
    case MLA_ERR_NOMEM: return "host allocation failed";
    default: break;
  }
  if (status <= MLA_ERR_HIP_BASE) return hipGetErrorString((hipError_t)(MLA_ERR_HIP_BASE - status));
  return "unknown status";
}

}  // extern "C"
