/*
 * mla_decode.h - C ABI of libmla_decode.so: split-KV (flash-decoding) MLA decode
 * attention over a paged FP8 E4M3 KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Operation. Each cached token is one 576-byte row of OCP FP8 E4M3 values: a 512-wide
 * latent followed by a 64-wide rope part; the cache is paged, 32 tokens per page; V is
 * the 512-wide latent of the same row (geometry and dtypes as in TensorRT-LLM issue
 * #20510 "CuTe DSL FP8 MLA decode slower after #19338", Setup). For request b with
 * KV length L_b and q_len query tokens, query token j attends causally to KV tokens
 * 0 .. L_b - q_len + j (the q = 8 "MTP verify" shape of the same Setup; q_len = 1 sees
 * all L_b). With s_i = softmax_scale * (q . K_i) over all 576 dims:
 *     O   = output_scale * sum_i exp(s_i) V_i / sum_i exp(s_i)      (BF16 out)
 *     LSE = ln sum_i exp(s_i)                                       (fp32 out)
 * softmax_scale and output_scale are the two scale arguments of the kernel module's
 * run() in that issue's Repro 1. LSE is the softmax statistic that the module can emit
 * (emit_softmax_stats, lse_dtype Float32 in the same listing); it excludes output_scale.
 *
 * Method. The host planner (mla_decode_plan) cuts each request's keys into S_b splits
 * of whole pages. mla_decode_partial runs one workgroup per (split, block of <= 96
 * query rows) and writes, per (row, split), an online-softmax partial (max, sum,
 * unnormalised O) in fp32; mla_decode_merge combines each row's partials, with groups of wavefronts
 * folding interleaved subsets of them and rescaling each group result by
 * 2^(group max - max) before the final combine (the KvSplit thread-group merge of
 * TensorRT-LLM PR #20380 "trtllm-gen FMHA: split the KV partials of a row across thread
 * groups in fmhaReductionKernel", Description, re-done for 64-wide wavefronts).
 * Splitting changes nothing beyond rounding: partial maxima are kept on integers (log2
 * units) so every rescale is an exact power of two.
 *
 * Layouts (all row-major, contiguous, device memory owned by the caller):
 *   q            uint8 E4M3 codes [B][q_len][H][576]
 *   kv_cache     uint8 E4M3 codes [num_pages][32][576]
 *   block_table  int32 [B][bt_stride]; entry p of request b is the cache page holding
 *                tokens 32p .. 32p+31; only entries p < ceil(L_b / 32) are read
 *   kv_lens      int32 [B] (device copy of the lengths given to the plan)
 *   o            BF16 [B][q_len][H][512]   (or fp32 for mla_decode_merge_f32)
 *   lse          fp32 [B][q_len][H]        (may be NULL)
 *   workspace    caller-allocated device scratch of mla_decode_workspace_size() bytes,
 *                256-byte aligned; it carries the partials from partial to merge
 * Flat row id: r = (b * q_len + j) * H + h.
 *
 * Threading and streams. A plan is immutable after creation and may be shared by
 * threads. All compute calls are asynchronous on `stream` (a hipStream_t; NULL = the
 * null stream), enqueue nothing else, and never synchronise the host. The library
 * allocates no device memory and throws nothing; its only global mutable state is the
 * per-GPU scratch array of mla_decode_noalloc (below).
 *
 * Errors. Every int-returning call returns MLA_OK (0) or a negative status. Argument,
 * shape and workspace checks run on the host before anything is enqueued, so a failed
 * call writes nothing. A HIP launch failure returns MLA_ERR_HIP_BASE - hipError_t.
 * Device-side preconditions that are not checked: block-table entries below
 * ceil(L_b / 32) must be valid page indices, and the device kv_lens should equal the
 * plan's. The kernels use min(device length, plan length): a smaller device length
 * leaves trailing splits empty (merged correctly), a larger one is cut to the plan's,
 * so no call reads a block-table entry beyond the ones the plan covers.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1)       /* null pointer, non-positive size, L_b < q_len, ... */
#define MLA_ERR_UNSUPPORTED_SHAPE (-2) /* outside the limits below */
#define MLA_ERR_WORKSPACE (-3)         /* workspace NULL, misaligned or too small */
#define MLA_ERR_NOMEM (-4)             /* host allocation of the plan failed */
#define MLA_ERR_HIP_BASE (-1000)       /* MLA_ERR_HIP_BASE - hipError_t */

#define MLA_D_QK 576      /* bytes per cached row: latent 512 + rope 64 */
#define MLA_D_V 512       /* latent width = V width = O width */
#define MLA_PAGE_SIZE 32  /* tokens per cache page */
#define MLA_MAX_BATCH 256 /* requests per plan */
#define MLA_MAX_ROWS_PER_REQUEST 4096 /* q_len * num_heads */
#define MLA_MAX_SPLIT_KV 1024         /* cap on splits per request */

#define MLA_KV_E4M3 0 /* q and cache hold OCP E4M3 codes: 576-byte rows */
#define MLA_KV_BF16 1 /* q and cache hold BF16 values: 1152-byte rows */

typedef struct mla_decode_plan_s mla_decode_plan_t;

/*
 * Build a split plan from the host copy of the KV lengths (the planner of the
 * per-request split plan in issue #20510, Repro 2, rewritten for 256 CUs).
 *   kv_lens_host  int32 [batch], each >= q_len
 *   split_kv > 0  uniform plan: every request gets min(split_kv, max_split_kv,
 *                 ceil(L_b / 32)) splits (the clamp of the plan to [1, split_kv]
 *                 described in that issue's follow-up comment);
 *   split_kv == 0 planner: splits per request in proportion to L_b so that all
 *                 (split, row block) work items fill num_cus CUs in one wave, capped at
 *                 max_split_kv (the issue raises that cap to 128 so that a single
 *                 request can occupy the whole GPU);
 *   max_split_kv  cap on splits per request, 1 .. MLA_MAX_SPLIT_KV (the issue uses 128
 *                 for 148 SMs; 256 lets one request fill the 256 CUs of an MI355X);
 *   num_cus       compute units to fill; 0 = query the current HIP device.
 * Every split holds a whole number of pages and none is empty. Splits are issued
 * longest request first. On success *out owns host memory freed by
 * mla_decode_plan_destroy.
 */
int mla_decode_plan(const int32_t* kv_lens_host, int32_t batch, int32_t q_len,
                    int32_t num_heads, int32_t split_kv, int32_t max_split_kv,
                    int32_t num_cus, mla_decode_plan_t** out);

/*
 * As mla_decode_plan, for a cache of the given element type (the BF16 kernel that
 * issue #20510, Repro 2, measures beside the FP8 one): kv_dtype MLA_KV_E4M3 (what
 * mla_decode_plan builds) or MLA_KV_BF16. With MLA_KV_BF16, q is BF16 [B][q_len][H][576]
 * (16-byte aligned) and the cache BF16 [P][32][576] (36,864-byte pages); every call that
 * takes q and kv_cache reads them with that type, the rest (block table, lengths,
 * workspace, O, LSE, epilogue options) is unchanged. BF16 rows are processed in blocks
 * of at most 32 query rows.
 */
int mla_decode_plan_ex(const int32_t* kv_lens_host, int32_t batch, int32_t q_len,
                       int32_t num_heads, int32_t split_kv, int32_t max_split_kv,
                       int32_t num_cus, int32_t kv_dtype, mla_decode_plan_t** out);

void mla_decode_plan_destroy(mla_decode_plan_t* plan);

/*
 * A copy of `plan` whose merge folds each row's partials with at most max_groups
 * wavefront groups (PR #20380, Description: the KvSplit width is an upper bound of 2, 4,
 * 8 or 16, or 1 for the serial fold, that the host halves until every group holds a
 * partial and the launch fits its budget). The copy's width is min(max_groups, the
 * planner's width); everything else is unchanged, so the partial pass is identical and
 * only the merge's summation order differs. max_groups: 1, 2, 4, 8 or 16, else
 * MLA_ERR_INVALID_ARG. Works for host and graph plans; *out is freed by
 * mla_decode_plan_destroy.
 */
int mla_decode_plan_with_merge_bound(const mla_decode_plan_t* plan, int32_t max_groups,
                                     mla_decode_plan_t** out);

/* Bytes of workspace the plan needs: fp32 partials, (512 + 4) * 4 bytes per (row,
 * split), and with split_workgroups > 1 (mla_decode_plan_get_info) as much again per
 * workgroup of a split for their states before the fold; graph plans also keep their
 * device plan at its head. 0 for a NULL plan. */
size_t mla_decode_workspace_size(const mla_decode_plan_t* plan);

/* Introspection, for tests and logs. splits/chunk_tokens may be NULL; otherwise they
 * receive S_b and the split length in tokens (a multiple of 32) per request. */
typedef struct {
  int32_t batch, q_len, num_heads;
  int32_t rows_per_request; /* q_len * num_heads */
  int32_t row_tiles;        /* row blocks (<= 96 rows each): workgroups per split */
  int32_t total_splits;     /* sum_b S_b */
  int32_t work_items;       /* total_splits * row_tiles */
  int32_t merge_groups;     /* wavefront groups per row in the merge (power of 2) */
  int32_t max_splits;       /* max_b S_b */
  int32_t merge_slices;     /* workgroups per row in the merge (1, 2, 4 or 8 slices of
                               the 512 output dims) */
  int32_t split_workgroups; /* workgroups per (split, row block) in the partial pass: 1,
                               or up to 8 when the plan has at most half as many work
                               items as CUs (host plans, and graph plans with a uniform
                               split_kv, by capacity); each takes a run of whole 64-token
                               steps of the split, and the pass folds their states into
                               the split's partial */
} mla_decode_plan_info_t;

int mla_decode_plan_get_info(const mla_decode_plan_t* plan, mla_decode_plan_info_t* info,
                             int32_t* splits, int32_t* chunk_tokens);

/*
 * Split-KV partial pass (issue #20510's FP8 split-KV kernel, redesigned for gfx950):
 * for every (request, split, row block) it gathers the split's pages into LDS with
 * 16-byte loads, forms QK^T on FP8 MFMA with fp32 accumulation, runs an exp2 online
 * softmax, and forms PV on FP8 MFMA with V read from the same LDS rows, writing fp32
 * partials to the workspace. softmax_scale is the fp32 scale on q . k. A plan whose
 * splits would leave CUs idle (split_workgroups > 1) runs each split on several
 * workgroups and folds their states in a second kernel; either way the workspace ends
 * with one partial per (split, row).
 */
int mla_decode_partial(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                       const int32_t* block_table, int64_t bt_stride,
                       const int32_t* kv_lens, float softmax_scale, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Merge pass (PR #20380's reduction, re-done for wavefronts): combines each row's
 * partials into O = output_scale * O / l, rounded to BF16 (nearest even), and
 * LSE = ln sum exp(s_i) in fp32 (skipped when lse is NULL). Empty partials (a split
 * in which a causal row sees no key) are skipped.
 */
int mla_decode_merge(const mla_decode_plan_t* plan, const void* workspace,
                     size_t workspace_bytes, float output_scale, void* o, float* lse,
                     void* stream);

/* As mla_decode_merge, but O is written as fp32 [B][q_len][H][512]: the values the
 * BF16 variant rounds. Used to compare results across split plans before rounding. */
int mla_decode_merge_f32(const mla_decode_plan_t* plan, const void* workspace,
                         size_t workspace_bytes, float output_scale, float* o, float* lse,
                         void* stream);

/* mla_decode_partial followed by mla_decode_merge on the same stream. */
int mla_decode(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
               const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
               float softmax_scale, float output_scale, void* workspace,
               size_t workspace_bytes, void* o, float* lse, void* stream);

/*
 * Ragged query batch (the module's is_var_q / query_lens in issue #20510, Repro 1):
 * as mla_decode with a plan built for q_len = the largest query count, plus
 *   q_lens  device int32 [batch]: query tokens of request b (clamped to [0, q_len]).
 * q, o and lse keep the [B][q_len][H] layout; query j < q_lens[b] of request b sees
 * keys [0, L_b - q_lens[b] + j] (the causal MTP rule with that request's count), and
 * rows j >= q_lens[b] come out as O = 0, LSE = -inf.
 */
int mla_decode_varq(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                    const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                    const int32_t* q_lens, float softmax_scale, float output_scale,
                    void* workspace, size_t workspace_bytes, void* o, float* lse,
                    void* stream);

/*
 * Graph path (the deployment setting of issue #20510, follow-up comments: under CUDA
 * graphs the KV lengths are not on the host, the scales come from device tensors, and
 * the kernel skips empty splits). Everything a call does is device work on `stream`
 * with no host read of device data, so a call can be captured in a HIP graph and
 * replayed while kv_lens and the scales change.
 *
 * mla_decode_plan_graph builds a plan from shapes and bounds only:
 *   max_kv_len    upper bound of every device length (>= 1); block-table rows must hold
 *                 ceil(max_kv_len / 32) entries (bt_stride);
 *   split_kv, max_split_kv, num_cus as for mla_decode_plan.
 * The workspace it asks for (mla_decode_workspace_size) is sized for the largest plan
 * any lengths <= max_kv_len can produce, plus the device plan at its head.
 * mla_decode_plan_get_info reports that capacity (splits and chunk_tokens are 0).
 *
 * mla_decode_graph runs three kernels: the device planner (the host planner's rules,
 * applied to kv_lens clamped to [0, max_kv_len]), the partial pass and the merge.
 *   kv_lens        int32 [batch], device; a request with length 0 (or shorter than
 *                  q_len, for the rows that see no key) yields O = 0 and LSE = -inf;
 *   q_lens         int32 [batch], device, or NULL: a ragged batch as in mla_decode_varq;
 *   softmax_scale  fp32 [1], device; output_scale fp32 [1], device;
 * other arguments as for mla_decode. Calls with a graph plan through mla_decode /
 * _partial / _merge (and the reverse) return MLA_ERR_INVALID_ARG.
 */
int mla_decode_plan_graph(int32_t batch, int32_t q_len, int32_t num_heads, int32_t max_kv_len,
                          int32_t split_kv, int32_t max_split_kv, int32_t num_cus,
                          mla_decode_plan_t** out);

/* Graph plan for a cache of the given element type (see mla_decode_plan_ex). */
int mla_decode_plan_graph_ex(int32_t batch, int32_t q_len, int32_t num_heads,
                             int32_t max_kv_len, int32_t split_kv, int32_t max_split_kv,
                             int32_t num_cus, int32_t kv_dtype, mla_decode_plan_t** out);

int mla_decode_graph(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                     const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                     const int32_t* q_lens, const float* softmax_scale,
                     const float* output_scale, void* workspace, size_t workspace_bytes,
                     void* o, float* lse, void* stream);

/*
 * Merge epilogue options: the steps after the combine in PR #20380 (Description:
 * sinks are applied after the groups are combined) and the MXFP8 output of the sparse
 * decode merge in PR #17441 "m3 decode perf clean" (commit messages: the merge emits
 * E4M3 values with UE8M0 block scales next to its BF16 O, identical to quantizing that
 * BF16 tensor afterwards). Each option is off when its pointer is NULL.
 *   sinks         device fp32 [H]: one sink logit per head, in the units of the scaled
 *                 scores; it joins the softmax denominator only:
 *                   O = output_scale * sum_i e^(s_i) v_i / (sum_i e^(s_i) + e^(sigma_h)),
 *                   LSE = ln(sum_i e^(s_i) + e^(sigma_h));
 *                 a row that sees no key gives O = 0, LSE = sigma_h.
 *   o_fp8         device uint8 [B][q_len][H][512], 8-byte aligned: E4M3 (OCP "fn")
 *                 codes of the BF16 O divided by its block scale, nearest even;
 *   o_fp8_scales  device uint8 [B][q_len][H][16]: one E8M0 scale (biased by 127) per 32
 *                 consecutive dims; 2^e with e the smallest integer such that the block's
 *                 largest |BF16 value| < 448 * 2^e (strictly: an amax of 1.75 * 2^k takes
 *                 the exponent above, as the commit message on the quantize tile states),
 *                 clamped to [-127, 127]. A block of scale byte 0 saturates (the commit
 *                 message on scale byte 0): its non-zero values are coded +-448 (0x7E with
 *                 the sign), its zeros stay zero codes.
 *                 o_fp8 and o_fp8_scales are given together or not at all.
 *   o             BF16 O as for mla_decode_merge; may be NULL when o_fp8 is given, and
 *                 must be 16-byte aligned when both are written.
 * The BF16 O, LSE and every other argument behave as in the call each variant extends.
 */
int mla_decode_merge_ex(const mla_decode_plan_t* plan, const void* workspace,
                        size_t workspace_bytes, float output_scale, const float* sinks, void* o,
                        float* lse, void* o_fp8, void* o_fp8_scales, void* stream);

/* mla_decode (q_lens NULL) or mla_decode_varq (q_lens given) with the epilogue options. */
int mla_decode_ex(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                  const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                  const int32_t* q_lens, float softmax_scale, float output_scale,
                  const float* sinks, void* workspace, size_t workspace_bytes, void* o,
                  float* lse, void* o_fp8, void* o_fp8_scales, void* stream);

/* mla_decode_graph with the epilogue options (sinks read from device memory at run time,
 * so they may change between replays of a captured call). */
int mla_decode_graph_ex(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                        const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                        const int32_t* q_lens, const float* softmax_scale,
                        const float* output_scale, const float* sinks, void* workspace,
                        size_t workspace_bytes, void* o, float* lse, void* o_fp8,
                        void* o_fp8_scales, void* stream);

/*
 * Key windows (kv_bounds, one of the run() arguments that issue #20510, Repro 1, lists
 * as added after #19338; the pages give it no description). Read here as one half-open
 * window of key positions per request that its queries are confined to, on top of the
 * causal rule:
 *   kv_bounds  device int32 [B][2] = (start_b, end_b): query j of request b sees the keys
 *              i with start_b <= i < end_b and i <= L_b - q_len_b + j. A negative start
 *              counts as 0, an end past L_b as L_b. Keys outside the window are never
 *              read: block-table entries of pages wholly outside it may hold anything,
 *              and cache slots of the window's first and last page outside it may hold
 *              anything, NaN codes included.
 *   A row with no visible key gives O = 0 and LSE = -inf (LSE = sigma_h with a sink).
 * Splits are planned from the lengths as without windows; a split wholly outside its
 * request's window does no work. The windows are read on the device at run time.
 *
 * mla_decode_partial_ex: mla_decode_partial with optional q_lens (as mla_decode_varq)
 * and kv_bounds (either may be NULL); merge its partials with any merge call.
 * mla_decode_bounded: mla_decode_ex with kv_bounds (not NULL).
 * mla_decode_graph_bounded: mla_decode_graph_ex with kv_bounds (not NULL).
 */
int mla_decode_partial_ex(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                          const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                          const int32_t* q_lens, const int32_t* kv_bounds, float softmax_scale,
                          void* workspace, size_t workspace_bytes, void* stream);

int mla_decode_bounded(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                       const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                       const int32_t* q_lens, const int32_t* kv_bounds, float softmax_scale,
                       float output_scale, const float* sinks, void* workspace,
                       size_t workspace_bytes, void* o, float* lse, void* o_fp8,
                       void* o_fp8_scales, void* stream);

int mla_decode_graph_bounded(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                             const int32_t* block_table, int64_t bt_stride,
                             const int32_t* kv_lens, const int32_t* q_lens,
                             const int32_t* kv_bounds, const float* softmax_scale,
                             const float* output_scale, const float* sinks, void* workspace,
                             size_t workspace_bytes, void* o, float* lse, void* o_fp8,
                             void* o_fp8_scales, void* stream);

/*
 * For callers that cannot allocate device memory or hand in a workspace: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * computation, checks and kernels as mla_decode with a host plan, except that the
 * partials live in a scratch array of MLA_NOALLOC_SCRATCH_BYTES (64 MiB) that the
 * library's code object holds on every GPU it runs on, until the process ends. The call
 * itself allocates nothing; its first call on a device looks up that device's array
 * (hipGetSymbolAddress) once.
 *   plan  a host plan (graph plans: MLA_ERR_INVALID_ARG) whose
 *         mla_decode_workspace_size() is at most MLA_NOALLOC_SCRATCH_BYTES, else
 *         MLA_ERR_WORKSPACE; every other argument as for mla_decode.
 * The current HIP device must be the one `stream` belongs to. Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on different streams,
 * or from different host threads) race and give undefined results; calls on one stream
 * are ordered and safe. Nothing in the array needs clearing between calls.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
int mla_decode_noalloc(const mla_decode_plan_t* plan, const void* q, const void* kv_cache,
                       const int32_t* block_table, int64_t bt_stride, const int32_t* kv_lens,
                       float softmax_scale, float output_scale, void* o, float* lse,
                       void* stream);

/* Static description of a status code (never NULL). */
const char* mla_decode_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
