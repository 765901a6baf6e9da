/*
 * pmqa.h - C ABI of the MI355X (gfx950) paged MQA logits library.
 *
 * The operation is the scoring step of a DeepSeek-style sparse-attention
 * indexer described on the page "[flashinfer] Blackwell 아키텍처를 위한
 * 고성능 Paged MQA Logits 커널 도입" (introduction: the indexer selects KV
 * tokens by a score that passes each head's query-key product through ReLU,
 * weights it per head and sums; an fp8 and an fp4 kernel).  For output
 * row r (query j of batch row b, r = b*next_n + j) and KV token t reached
 * through the block table:
 *
 *     logits[r, t] = sum_h w[r, h] * ReLU(scale_t * dot(q[r, h, :], k_t))
 *                                        for t <  ctx_b - next_n + 1 + j
 *     logits[r, t] = -inf                for the other t < max_context_len
 *
 * Work is cut into 256-token units of one batch row and spread over a
 * persistent grid by a schedule computed on the GPU (sections 1 and 2 of the
 * same page: binary search over per-row unit counts, zero-length rows
 * skipped, no host round trip so the pair of calls can be graph-captured).
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - Pointers are DEVICE pointers unless stated otherwise.  Every buffer is
 *    owned by the caller; the library never allocates, frees or retains one.
 *  - Calls are asynchronous on `stream` and never synchronize the host,
 *    except in validate mode (below).  No call allocates device memory, so
 *    compute_schedule followed by a logits call can be captured into a HIP
 *    graph and replayed.
 *  - No C++ exception crosses the ABI.  Every call returns a pmqa_status_t;
 *    pmqa_last_error() returns a message naming the offending argument.
 *  - Always-on checks cost O(1) host work: null pointers, alignment, sizes,
 *    strides, the compiled specialisation (num_heads 64, 32 or 16, head_dim
 *    128, page_size 64, next_n 1 or 2) and, once per device, that the device
 *    is a gfx950.
 *  - Validate mode (environment variable PMQA_VALIDATE_INPUTS=1, read on
 *    every call) adds checks of device contents: context lengths, the used
 *    block-table entries and the schedule's freshness.  They copy data to the
 *    host and synchronize `stream`, so validate mode refuses a capturing
 *    stream with PMQA_ERR_CAPTURING.
 *  - Without validate mode, out-of-range device contents never make the
 *    kernels read or write outside the buffers described here (indices are
 *    clamped), but the results are then unspecified.
 */
#ifndef PMQA_H
#define PMQA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Compiled specialisation. */
#define PMQA_NUM_HEADS 64
#define PMQA_HEAD_DIM 128
#define PMQA_PAGE_SIZE 64
#define PMQA_UNIT_TOKENS 256 /* one schedule work unit = 4 pages of one row */
#define PMQA_FP8_PAGE_BYTES 8448 /* 64*128 e4m3fn + 64 fp32 scales */
#define PMQA_FP4_PAGE_BYTES 4352 /* 64*64 packed e2m1 + 64*4 e8m0 */

typedef enum {
  PMQA_OK = 0,
  PMQA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size or stride */
  PMQA_ERR_UNSUPPORTED = 2,      /* not a gfx950 device, or shape not compiled */
  PMQA_ERR_INVALID_VALUE = 3,    /* validate mode: bad context length or page id */
  PMQA_ERR_STALE_SCHEDULE = 4,   /* validate mode: schedule does not match inputs */
  PMQA_ERR_CAPTURING = 5,        /* validate mode on a capturing stream */
  PMQA_ERR_HIP = 6               /* a HIP runtime call failed */
} pmqa_status_t;

typedef enum { PMQA_VARIANT_FP8 = 0, PMQA_VARIANT_FP4 = 1 } pmqa_variant_t;

/* Element type of the K values given to the quantize_append calls. */
typedef enum { PMQA_DTYPE_F32 = 0, PMQA_DTYPE_BF16 = 1 } pmqa_dtype_t;

/* Message of the last failing call on this thread ("" after success).  The
 * string is owned by the library and valid until the next call on the
 * thread. */
const char* pmqa_last_error(void);

/* Persistent-grid size W of the fp8 logits kernel with next_n 1 and 64 heads
 * (the batch decode kernel) on `device`: three quarters of (compute units
 * times its resident workgroups per compute unit), times 4 wavefronts per
 * workgroup (one worker = one wavefront; the value of
 * pmqa_default_num_workers for this kernel).  Host-only query.  Returns -1 on failure (not a gfx950
 * device, or a HIP error; pmqa_last_error() says which).
 *
 * Page: section 2 (a persistent grid whose work partition is computed per
 * call).  Any W >= 1 gives bitwise-identical logits; W only sets how many
 * workers share the units.  The other kernels' best W differs (MXFP4 runs
 * two wavefronts per SIMD): pmqa_default_num_workers gives it per variant. */
int pmqa_num_workers(int device);

/* Persistent-grid size for a logits kernel on `device`: compute units times
 * the kernel's resident workgroups per compute unit, times 4 wavefronts per
 * workgroup (one worker = one wavefront), except that the fp8 kernel with
 * next_n 1 takes three quarters of those workgroups (it streams K faster
 * with fewer readers; the next_n 2 and MXFP4 kernels, with twice the MFMA
 * and epilogue work per byte, are fastest with all of them).  The kernel,
 * and so its occupancy, depends on variant, next_n and num_heads (64, 32 or
 * 16).  Host-only query; writes the count to *num_workers (host pointer). */
pmqa_status_t pmqa_default_num_workers(int device, int32_t variant, int32_t next_n,
                                       int32_t num_heads, int32_t* num_workers);

/* Bytes of a schedule buffer for `batch` rows and `num_workers` workers:
 * 4 * (8 + 2*(num_workers+1) + batch + 1).  Returns 0 for invalid sizes. */
size_t pmqa_schedule_bytes(int32_t batch, int32_t num_workers);

/*
 * compute_schedule - per-call persistent-worker partition, on the GPU.
 *
 * Page: sections 1-2 (linear partition scan replaced by a binary search;
 * schedule computed on the GPU so it can be graph-captured) and the general
 * lessons (a schedule stays valid only while every ceil(context_len/256) is
 * unchanged).
 *
 *   context_lens  int32 [batch]; lengths < 0 count as 0 units.
 *   batch         >= 1.
 *   num_workers   >= 1; must equal the value later passed to the logits call.
 *   schedule      int32 buffer of pmqa_schedule_bytes(batch, num_workers)
 *                 bytes, 4-byte aligned, written entirely:
 *     [0] magic 0x41514D50, [1] batch, [2] num_workers, [3] total units T
 *         (-1 if T would exceed 2^31-1; the logits calls then write only
 *         -inf), [4] unit tokens (256), [5..7] zero;
 *     [8 + 2w], [9 + 2w]  start (row, unit) of worker w, w = 0..num_workers;
 *         worker w owns global units [floor(w*T/W), floor((w+1)*T/W)) of the
 *         row-major sequence of (row, unit) pairs; a start never names a row
 *         with zero units; worker num_workers starts at (batch, 0);
 *     [10 + 2*num_workers + b]  exclusive prefix sum S[b] of
 *         c_b = ceil(context_lens[b]/256), b = 0..batch.
 *
 * One workgroup; no host synchronization.
 */
pmqa_status_t compute_schedule(const int32_t* context_lens, int32_t batch, int32_t num_workers,
                               int32_t* schedule, hipStream_t stream);

/*
 * compute_schedule_linear - the same schedule, each worker's start found by
 * a linear scan of the prefix sums.
 *
 * Page: section 1, third bullet: the partition search before the change was
 * a linear scan, and at batch 2048 the binary search cut the runtime launch
 * cost tenfold.  The result is identical to compute_schedule's word for
 * word; this entry point exists to measure that cost on the same device.
 * Arguments, buffer layout, errors and graph capture as compute_schedule.
 */
pmqa_status_t compute_schedule_linear(const int32_t* context_lens, int32_t batch,
                                      int32_t num_workers, int32_t* schedule,
                                      hipStream_t stream);

/*
 * refresh_schedule - reuse a schedule while it is still valid, rebuild it
 * on the device when it is not.
 *
 * Page: general lessons, first item (schedule metadata may be reused, but
 * must be recomputed whenever some ceil(context_len/256) changes) and the
 * reviewer feedback (stale metadata under graph reuse; recompute when a
 * length crosses a 256-token boundary).
 *
 *   context_lens, batch, num_workers   as compute_schedule.
 *   schedule      int32 buffer of pmqa_schedule_bytes(batch, num_workers)
 *                 bytes: read, and rewritten only when stale.  It is kept
 *                 as is when its header holds the magic, this batch and
 *                 num_workers, unit 256 and T = S[batch], S[0] = 0, and
 *                 S[b+1] - S[b] = ceil(context_lens[b]/256) for every row;
 *                 otherwise it is rebuilt with exactly the contents
 *                 compute_schedule writes.  The worker starts are not
 *                 re-checked: a buffer last written by compute_schedule (or
 *                 by this call) for the same batch and num_workers is valid
 *                 whenever those checks pass.
 *   recomputed    NULL, or a device int32 that receives 1 when the buffer
 *                 was rebuilt and 0 when it was kept (4-byte aligned).
 *
 * One workgroup; no host synchronization; can be captured into a graph and
 * replayed as lengths grow.  Errors as compute_schedule.
 */
pmqa_status_t refresh_schedule(const int32_t* context_lens, int32_t batch, int32_t num_workers,
                               int32_t* schedule, int32_t* recomputed, hipStream_t stream);

/*
 * paged_mqa_logits_fp8 - logits from an fp8 paged K cache.
 *
 * Page: introduction (fp8 kernel, head scores through ReLU, weighted, summed) and
 * section 1 (zero-length rows skipped by the task iterator; an epilogue
 * sized by num_heads).
 *
 *   q             e4m3fn [batch, next_n, H, 128], contiguous, 16-B aligned
 *                 (H = num_heads).
 *   kv_cache      uint8 [num_pages][8448], 16-B aligned: per page 64 tokens x
 *                 128 e4m3fn bytes (token-major), then 64 little-endian fp32
 *                 per-token scales.  Only pages of tokens t < ctx_b are read.
 *   weights       fp32 [batch*next_n, H], contiguous, 16-B aligned.
 *   context_lens  int32 [batch].
 *   block_table   int32 [batch, block_table_stride]; entry i of row b names
 *                 the physical page of tokens [64i, 64i+64).  Only entries
 *                 i < ceil(ctx_b/64) are used (others of the row may be read).
 *   schedule      from compute_schedule(context_lens, batch, num_workers).
 *   logits        fp32 [batch*next_n, logits_stride], 16-B aligned,
 *                 logits_stride % 4 == 0 and >= max_context_len.  Row
 *                 r = b*next_n + j gets columns [0, max_context_len): the
 *                 scores for t < min(ctx_b - next_n + 1 + j, max_context_len)
 *                 and -inf for the rest (tokens >= max_context_len are
 *                 truncated).  Columns >= max_context_len are not touched.
 *   num_heads 64, 32 or 16, head_dim 128, page_size 64, next_n 1 or 2 (else
 *   PMQA_ERR_UNSUPPORTED); num_pages >= 1; block_table_stride >= 1;
 *   max_context_len >= 1.
 */
pmqa_status_t paged_mqa_logits_fp8(const void* q, const void* kv_cache, const float* weights,
                                   const int32_t* context_lens, const int32_t* block_table,
                                   const int32_t* schedule, float* logits, int32_t batch,
                                   int32_t next_n, int32_t num_heads, int32_t head_dim,
                                   int32_t page_size, int64_t num_pages,
                                   int32_t block_table_stride, int32_t max_context_len,
                                   int64_t logits_stride, int32_t num_workers,
                                   hipStream_t stream);

/*
 * paged_mqa_logits_fp4 - logits from an MXFP4 paged K cache.
 *
 * Page: introduction (fp4 kernel).  Elements are OCP MXFP4: E2M1 values with
 * one E8M0 scale per 32 consecutive elements along head_dim; there is no
 * per-token fp32 scale (scale_t = 1).
 *
 *   q             packed e2m1 [batch, next_n, H, 64] (element 2i in the low
 *                 nibble of byte i), 16-B aligned.
 *   q_scale       e8m0 [batch, next_n, H, 4] (no alignment requirement).
 *   kv_cache      uint8 [num_pages][4352], 16-B aligned: 64 tokens x 64 packed
 *                 bytes (token-major), then 64 tokens x 4 e8m0 block scales.
 *   All other arguments as for paged_mqa_logits_fp8.
 */
pmqa_status_t paged_mqa_logits_fp4(const void* q, const void* q_scale, const void* kv_cache,
                                   const float* weights, const int32_t* context_lens,
                                   const int32_t* block_table, const int32_t* schedule,
                                   float* logits, int32_t batch, int32_t next_n,
                                   int32_t num_heads, int32_t head_dim, int32_t page_size,
                                   int64_t num_pages, int32_t block_table_stride,
                                   int32_t max_context_len, int64_t logits_stride,
                                   int32_t num_workers, hipStream_t stream);

/*
 * select_topk - the k largest logits of each row, by column.
 *
 * Page: introduction (the logits feed the indexer, which selects KV tokens
 * by them).  The page gives neither k nor an order; the rule here: row r's
 * candidates are its first lengths[r] columns (clamped to
 * [0, max_context_len]); the selection is the k largest candidates in the
 * total order of fp32 values where -0 < +0, equal values ordered by column,
 * lower first (NaN has no place in the order: rows holding NaN get an
 * unspecified selection); the selected columns are written in ascending
 * order, with their values.  A row with fewer than k candidates writes all
 * of them and pads with column -1 and value -inf.
 *
 *   logits          fp32 [rows, logits_stride], 16-byte aligned; only the
 *                   candidate columns are read.
 *   logits_stride   >= max_context_len, multiple of 4.
 *   rows            >= 1.
 *   lengths         int32 [rows] candidate counts.
 *   k               >= 1.
 *   topk_indices    int32 [rows, topk_stride], 4-byte aligned; columns
 *                   [0, k) written.
 *   topk_values     fp32 [rows, topk_stride] or NULL.
 *   topk_stride     >= k.
 *   select_workspace        NULL, or a device buffer of at least
 *                   pmqa_select_workspace_bytes(rows, max_context_len, k)
 *                   bytes, 16-byte aligned, owned by the caller, contents
 *                   unspecified before and after the call (error
 *                   PMQA_ERR_INVALID_ARGUMENT when smaller or misaligned).  With it, and at most 512 rows,
 *                   the rows too long to be kept in LDS are split into
 *                   chunks over many workgroups (two more kernels run
 *                   first); the result is the same.  Calls that share one
 *                   workspace must be ordered (one stream).
 *   select_workspace_bytes  its size.
 *
 * One kernel (two more with the split workspace): rows of at most 6144
 * candidates are selected by one wavefront each, longer rows by one
 * workgroup each (when every row gets a workgroup at once, at most two
 * rows per compute unit, every row of more than k candidates gets one); no
 * host synchronization; can be graph-captured.
 */
pmqa_status_t select_topk(const float* logits, int64_t logits_stride, int32_t rows,
                          int32_t max_context_len, const int32_t* lengths, int32_t k,
                          int32_t* topk_indices, float* topk_values, int64_t topk_stride,
                          void* select_workspace, size_t select_workspace_bytes,
                          hipStream_t stream);

/*
 * select_topk_noalloc - select_topk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same selection, bit for bit, with the split
 * workspace taken from a static scratch array of the library instead of a
 * caller's buffer.  It allocates nothing: the array is part of the loaded
 * code object, one copy per device (about 24.6 MiB, held until the process
 * ends), enough for every call select_topk would split (at most 512 rows);
 * a call needing more (not possible with the current sizes) returns
 * PMQA_ERR_INVALID_ARGUMENT.
 *
 * Every call on a device shares that device's scratch, and the scratch keeps
 * the last call's contents (no call depends on them).  Calls that may
 * overlap on one device (different streams, or several host threads
 * without ordering) race on it: order them on one stream.
 *
 * Arguments, results and errors as select_topk, without the workspace.
 */
pmqa_status_t select_topk_noalloc(const float* logits, int64_t logits_stride, int32_t rows,
                                  int32_t max_context_len, const int32_t* lengths, int32_t k,
                                  int32_t* topk_indices, float* topk_values,
                                  int64_t topk_stride, hipStream_t stream);

/*
 * pmqa_select_workspace_bytes - bytes of the optional select_workspace of
 * select_topk and paged_mqa_topk_fp8/fp4 for `rows` rows of at most
 * max_context_len candidates and this k (about 49 KB per row); 0 when no
 * workspace would be used: rows < 1 or rows > 512, or no row can be too
 * long for one workgroup's LDS (max_context_len <= 7680 or <= k).
 * Host-only arithmetic.
 */
size_t pmqa_select_workspace_bytes(int32_t rows, int32_t max_context_len, int32_t k);

/*
 * paged_mqa_topk_fp8 / paged_mqa_topk_fp4 - the indexer step: logits of
 * every scheduled unit, then the top k per output row.
 *
 * Same inputs, schedule and errors as paged_mqa_logits_fp8 / _fp4, with
 * logits_workspace in place of the logits output: on return it holds the
 * logits of every scheduled unit's columns (columns [0, 256*c_b) of the
 * rows of batch row b, c_b its unit count in the schedule; -inf past a
 * row's causal limit) and unspecified values elsewhere (no -inf fill is
 * written).  Row r = b*next_n + j then selects as select_topk with
 * lengths[r] = min(ctx_b - next_n + 1 + j, 256*c_b, max_context_len)
 * (at least 0; 0 for every row when the schedule header does not describe
 * the call).
 *
 *   k, topk_indices, topk_values, topk_stride, select_workspace,
 *   select_workspace_bytes   as select_topk, with batch*next_n rows.
 */
pmqa_status_t paged_mqa_topk_fp8(const void* q, const void* kv_cache, const float* weights,
                                 const int32_t* context_lens, const int32_t* block_table,
                                 const int32_t* schedule, float* logits_workspace, int32_t k,
                                 int32_t* topk_indices, float* topk_values, int64_t topk_stride,
                                 void* select_workspace, size_t select_workspace_bytes,
                                 int32_t batch, int32_t next_n, int32_t num_heads,
                                 int32_t head_dim, int32_t page_size, int64_t num_pages,
                                 int32_t block_table_stride, int32_t max_context_len,
                                 int64_t logits_stride, int32_t num_workers, hipStream_t stream);
pmqa_status_t paged_mqa_topk_fp4(const void* q, const void* q_scale, const void* kv_cache,
                                 const float* weights, const int32_t* context_lens,
                                 const int32_t* block_table, const int32_t* schedule,
                                 float* logits_workspace, int32_t k, int32_t* topk_indices,
                                 float* topk_values, int64_t topk_stride, void* select_workspace,
                                 size_t select_workspace_bytes, int32_t batch,
                                 int32_t next_n, int32_t num_heads, int32_t head_dim,
                                 int32_t page_size, int64_t num_pages,
                                 int32_t block_table_stride, int32_t max_context_len,
                                 int64_t logits_stride, int32_t num_workers, hipStream_t stream);

/*
 * quantize_append_fp8 / quantize_append_fp4 - quantize new K tokens and
 * write them into the paged cache the logits calls read.
 *
 * Page: introduction (the fp8 and fp4 paged K caches the two kernels
 * consume).  The page does not say how the cache is written; these calls
 * use the plainest rules of the two formats:
 *   fp8:   per token, scale = amax/448 (fp32, nearest even) stored as the
 *          token's fp32 scale; each value becomes the E4M3fn byte nearest
 *          to x/scale (|x/scale| clamped to 448), ties to the even code,
 *          sign bit = sign of x/scale; an all-zero token gets scale 0 and
 *          zero bytes.
 *   MXFP4: per 32 values, e = floor(log2 amax) - 2 clamped to [-127, 127],
 *          stored as the E8M0 byte e+127 (0 for an all-zero block); each
 *          value becomes the E2M1 code nearest to |x|*2^-e, ties to the even
 *          code, saturating at 6, sign bit only on a non-zero magnitude;
 *          value 2i is the low nibble of byte i.
 *
 *   k             [num_tokens, head_dim] row-major values of type k_dtype
 *                 (PMQA_DTYPE_F32 or PMQA_DTYPE_BF16), 16-byte aligned,
 *                 finite.
 *   num_tokens    >= 0 (0: nothing is read or written).
 *   head_dim      must be 128.
 *   slot_mapping  int64 [num_tokens], 8-byte aligned: token i goes to page
 *                 slot/64, row slot%64.  A negative slot skips the token;
 *                 a slot at or past num_pages*64 is skipped too (validate
 *                 mode reports it as PMQA_ERR_INVALID_VALUE).  Slots must be
 *                 distinct (validate mode checks); two tokens with one slot
 *                 leave that row unspecified.
 *   kv_cache      [num_pages][PMQA_FP8_PAGE_BYTES] (fp8) or
 *                 [num_pages][PMQA_FP4_PAGE_BYTES] (fp4) bytes, 16-byte
 *                 aligned; only the rows and scales of the given slots are
 *                 written.
 *
 * One wavefront per token; no host synchronization outside validate mode;
 * can be captured into a graph.
 */
pmqa_status_t quantize_append_fp8(const void* k, int32_t k_dtype, int64_t num_tokens,
                                  int32_t head_dim, const int64_t* slot_mapping, void* kv_cache,
                                  int64_t num_pages, hipStream_t stream);
pmqa_status_t quantize_append_fp4(const void* k, int32_t k_dtype, int64_t num_tokens,
                                  int32_t head_dim, const int64_t* slot_mapping, void* kv_cache,
                                  int64_t num_pages, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PMQA_H */
