// C-ABI entry points of the paged MQA logits library (declared in pmqa.h).
//
// Argument checks follow the page "[flashinfer] Blackwell 아키텍처를 위한 고성능
// Paged MQA Logits 커널 도입" (why-it-matters section and reviewer feedback:
// optional input validation at the API boundary; the schedule must be
// recomputed whenever a context length crosses a 256-token boundary).  Every
// check that needs only host data is always on; checks of device contents
// run in validate mode (PMQA_VALIDATE_INPUTS=1) because they synchronize.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include "pmqa.h"
#include "pmqa_internal.h"

namespace {

thread_local char g_err[512] = "";

pmqa_status_t fail(pmqa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

pmqa_status_t ok() {
  g_err[0] = '\0';
  return PMQA_OK;
}

constexpr int kMaxDevices = 64;
// 0 = not checked, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch[kMaxDevices];
// compute units per device (0 = not queried yet)
std::atomic<int> g_cus[kMaxDevices];

pmqa_status_t check_device(int* dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PMQA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(PMQA_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                     std::memory_order_release);
    g_arch[dev].store(st, std::memory_order_release);
  }
  if (st != 1) return fail(PMQA_ERR_UNSUPPORTED, "device %d is not a gfx950 (MI355X)", dev);
  if (dev_out) *dev_out = dev;
  return PMQA_OK;
}

bool validate_mode() {
  const char* v = getenv("PMQA_VALIDATE_INPUTS");
  return v && v[0] && strcmp(v, "0") != 0;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Outputs up to this size are filled by the unit kernel's workers.
constexpr int64_t kTailFillInKernelBytes = 32ll << 20;

int64_t sched_words(int64_t batch, int64_t workers) {
  return pmqa::kSchedHeader + 2 * (workers + 1) + batch + 1;
}

struct Shape {
  int32_t batch, next_n, bt_stride, max_ctx, workers;
  int64_t num_pages, ldo;
};

pmqa_status_t check_shape(const Shape& s, int32_t num_heads, int32_t head_dim, int32_t page_size) {
  if (s.batch < 1) return fail(PMQA_ERR_INVALID_ARGUMENT, "batch = %d must be >= 1", s.batch);
  if ((num_heads != 64 && num_heads != 32 && num_heads != 16) || head_dim != pmqa::kHeadDim ||
      page_size != pmqa::kPage)
    return fail(PMQA_ERR_UNSUPPORTED,
                "(num_heads, head_dim, page_size) = (%d, %d, %d) not compiled; only "
                "(64, 32 or 16, 128, 64)",
                num_heads, head_dim, page_size);
  if (s.next_n != 1 && s.next_n != 2)
    return fail(PMQA_ERR_UNSUPPORTED, "next_n = %d not compiled; only 1 or 2", s.next_n);
  if (s.num_pages < 1)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "num_pages = %lld must be >= 1", (long long)s.num_pages);
  if (s.bt_stride < 1)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "block_table_stride = %d must be >= 1", s.bt_stride);
  if (s.max_ctx < 1 || s.max_ctx > (1 << 29))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "max_context_len = %d must be in [1, 2^29]", s.max_ctx);
  if (s.ldo < s.max_ctx)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "logits_stride = %lld < max_context_len = %d",
                (long long)s.ldo, s.max_ctx);
  if (s.ldo % 4 != 0)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "logits_stride = %lld must be a multiple of 4",
                (long long)s.ldo);
  if (s.workers < 1)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "num_workers = %d must be >= 1", s.workers);
  if ((int64_t)s.batch * s.next_n > INT32_MAX / pmqa::kHeads)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "batch*next_n = %lld too large",
                (long long)s.batch * s.next_n);
  return PMQA_OK;
}

// Validate mode: device contents, read back to the host.
pmqa_status_t validate_contents(const int32_t* ctx, const int32_t* bt, const int32_t* sched,
                                const Shape& s, hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
  if (cap != hipStreamCaptureStatusNone)
    return fail(PMQA_ERR_CAPTURING, "PMQA_VALIDATE_INPUTS is set but the stream is capturing");
  std::vector<int32_t> hctx(s.batch);
  std::vector<int32_t> hbt((size_t)s.batch * s.bt_stride);
  std::vector<int32_t> hs(sched_words(s.batch, s.workers));
  e = hipMemcpyAsync(hctx.data(), ctx, hctx.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(hbt.data(), bt, hbt.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(hs.data(), sched, hs.size() * 4, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "validate copy: %s", hipGetErrorString(e));
  const int32_t* S = hs.data() + pmqa::kSchedHeader + 2 * (s.workers + 1);
  if (hs[0] != pmqa::kSchedMagic || hs[1] != s.batch || hs[2] != s.workers)
    return fail(PMQA_ERR_STALE_SCHEDULE,
                "schedule header (magic %08x, batch %d, workers %d) does not match the call "
                "(batch %d, workers %d)",
                (unsigned)hs[0], hs[1], hs[2], s.batch, s.workers);
  if (hs[3] < 0)
    return fail(PMQA_ERR_INVALID_VALUE, "total work units exceed 2^31-1");
  for (int32_t b = 0; b < s.batch; ++b) {
    const int32_t L = hctx[b];
    if (L < 0) return fail(PMQA_ERR_INVALID_VALUE, "context_lens[%d] = %d < 0", b, L);
    const int64_t pages = ((int64_t)L + pmqa::kPage - 1) / pmqa::kPage;
    if (pages > s.bt_stride)
      return fail(PMQA_ERR_INVALID_VALUE,
                  "context_lens[%d] = %d needs %lld pages > block_table_stride %d", b, L,
                  (long long)pages, s.bt_stride);
    const int32_t c = (int32_t)(((int64_t)L + pmqa::kUnit - 1) / pmqa::kUnit);
    if (S[b + 1] - S[b] != c)
      return fail(PMQA_ERR_STALE_SCHEDULE,
                  "schedule is stale: row %d has %d units, context_lens[%d] = %d needs %d "
                  "(recompute the schedule when ceil(context_len/256) changes)",
                  b, S[b + 1] - S[b], b, L, c);
    const int64_t used = pages < s.bt_stride ? pages : s.bt_stride;
    for (int64_t i = 0; i < used; ++i) {
      const int32_t pid = hbt[(size_t)b * s.bt_stride + i];
      if (pid < 0 || pid >= s.num_pages)
        return fail(PMQA_ERR_INVALID_VALUE, "block_table[%d, %lld] = %d outside [0, %lld)", b,
                    (long long)i, pid, (long long)s.num_pages);
    }
  }
  return PMQA_OK;
}

// fill: -inf over the columns no unit writes (the logits calls); the top-k
// calls skip it, their selection reads only the columns the units write.
pmqa_status_t logits_common(int variant, const void* q, const void* q_scale, const void* kv,
                            const float* weights, const int32_t* ctx, const int32_t* bt,
                            const int32_t* sched, float* logits, const Shape& s,
                            int32_t num_heads, int32_t head_dim, int32_t page_size,
                            hipStream_t stream, bool fill = true) {
  if (!q) return fail(PMQA_ERR_INVALID_ARGUMENT, "q is null");
  if (variant == PMQA_VARIANT_FP4 && !q_scale)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "q_scale is null");
  if (!kv) return fail(PMQA_ERR_INVALID_ARGUMENT, "kv_cache is null");
  if (!weights) return fail(PMQA_ERR_INVALID_ARGUMENT, "weights is null");
  if (!ctx) return fail(PMQA_ERR_INVALID_ARGUMENT, "context_lens is null");
  if (!bt) return fail(PMQA_ERR_INVALID_ARGUMENT, "block_table is null");
  if (!sched) return fail(PMQA_ERR_INVALID_ARGUMENT, "schedule is null");
  if (!logits) return fail(PMQA_ERR_INVALID_ARGUMENT, "logits is null");
  if (!aligned(q, 16)) return fail(PMQA_ERR_INVALID_ARGUMENT, "q must be 16-byte aligned");
  if (!aligned(kv, 16)) return fail(PMQA_ERR_INVALID_ARGUMENT, "kv_cache must be 16-byte aligned");
  if (!aligned(weights, 16))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "weights must be 16-byte aligned");
  if (!aligned(logits, 16))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "logits must be 16-byte aligned");
  if (!aligned(ctx, 4) || !aligned(bt, 4) || !aligned(sched, 4))
    return fail(PMQA_ERR_INVALID_ARGUMENT,
                "context_lens, block_table and schedule must be 4-byte aligned");
  pmqa_status_t st = check_shape(s, num_heads, head_dim, page_size);
  if (st != PMQA_OK) return st;
  int dev = 0;
  st = check_device(&dev);
  if (st != PMQA_OK) return st;
  if (validate_mode()) {
    st = validate_contents(ctx, bt, sched, s, stream);
    if (st != PMQA_OK) return st;
  }
  pmqa::LogitsArgs a;
  a.q = static_cast<const uint8_t*>(q);
  a.q_scale = static_cast<const uint8_t*>(q_scale);
  a.kv = static_cast<const uint8_t*>(kv);
  a.weights = weights;
  a.ctx = ctx;
  a.bt = bt;
  a.sched = sched;
  a.out = logits;
  a.num_pages = s.num_pages;
  a.ldo = s.ldo;
  a.batch = s.batch;
  a.bt_stride = s.bt_stride;
  a.max_ctx = s.max_ctx;
  a.num_workers = s.workers;
  a.flush_ticks = 1;  // replaced by the launcher
  // Small outputs get their -inf past the units from the unit kernel's own
  // workers, which saves the fill kernel's launch and its pass over the
  // output (measured on MI355X: mid_fp8, 8 MB of output, call 42 -> 39 us);
  // large ones keep the separate sweep, whose dense write stream is faster
  // than stores mixed into the K stream.
  const int64_t out_rows = (int64_t)s.batch * s.next_n;
  a.fill_tails = fill && out_rows <= s.workers &&
                 out_rows * s.max_ctx * 4 <= kTailFillInKernelBytes;
  hipError_t e = hipSuccess;
  if (fill && !a.fill_tails) {
    e = pmqa::launch_neg_inf_fill(logits, s.ldo, (int64_t)s.batch * s.next_n, s.max_ctx,
                                  g_cus[dev].load(std::memory_order_acquire), stream);
    if (e != hipSuccess) return fail(PMQA_ERR_HIP, "-inf fill launch: %s", hipGetErrorString(e));
  }
  e = variant == PMQA_VARIANT_FP8 ? pmqa::launch_logits_fp8(a, s.next_n, num_heads, stream)
                                  : pmqa::launch_logits_fp4(a, s.next_n, num_heads, stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "logits launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* pmqa_last_error(void) { return g_err; }

size_t pmqa_schedule_bytes(int32_t batch, int32_t num_workers) {
  if (batch < 1 || num_workers < 1) return 0;
  return (size_t)sched_words(batch, num_workers) * sizeof(int32_t);
}

pmqa_status_t pmqa_default_num_workers(int device, int32_t variant, int32_t next_n,
                                       int32_t num_heads, int32_t* num_workers) {
  if (!num_workers) return fail(PMQA_ERR_INVALID_ARGUMENT, "num_workers is null");
  if (variant != PMQA_VARIANT_FP8 && variant != PMQA_VARIANT_FP4)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "variant = %d is not fp8 (0) or fp4 (1)", variant);
  if (next_n != 1 && next_n != 2)
    return fail(PMQA_ERR_UNSUPPORTED, "next_n = %d not compiled; only 1 or 2", next_n);
  if (num_heads != 64 && num_heads != 32 && num_heads != 16)
    return fail(PMQA_ERR_UNSUPPORTED, "num_heads = %d not compiled; only 64, 32 or 16",
                num_heads);
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (device != cur) {
    e = hipSetDevice(device);
    if (e != hipSuccess) return fail(PMQA_ERR_HIP, "hipSetDevice(%d): %s", device, hipGetErrorString(e));
  }
  pmqa_status_t st = check_device(nullptr);
  int cus = 0, blocks = 0;
  if (st == PMQA_OK) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess) e = pmqa::logits_blocks_per_cu(variant, next_n, num_heads, &blocks);
    if (e != hipSuccess) st = fail(PMQA_ERR_HIP, "occupancy query: %s", hipGetErrorString(e));
  }
  if (device != cur) hipSetDevice(cur);
  if (st != PMQA_OK) return st;
  if (blocks < 1) blocks = 1;
  int64_t groups = (int64_t)cus * blocks;
  // The fp8 kernel with one query row per batch row streams K faster with
  // fewer readers: three quarters of the workgroups that fit (measured on
  // MI355X, B = 2048 decode: 768 workers 315 us per call, 1024 workers 323
  // us; a plain gather of the same pages 6.89 against 6.82 TB/s).  Its
  // next_n = 2 kernel and the MXFP4 kernel, with twice the MFMA and epilogue
  // work per byte, are fastest with every workgroup (1024 workers 457 us
  // against 768 workers 512 us for B = 256, next_n = 2).
  if (variant == PMQA_VARIANT_FP8 && next_n == 1 && groups >= 8) groups = groups * 3 / 4;
  *num_workers = (int32_t)(groups * pmqa::kWavesPerBlock);
  return ok();
}

int pmqa_num_workers(int device) {
  int32_t w = 0;
  if (pmqa_default_num_workers(device, PMQA_VARIANT_FP8, 1, 64, &w) != PMQA_OK) return -1;
  return w;
}

namespace {

pmqa_status_t check_schedule_args(const int32_t* context_lens, int32_t batch,
                                  int32_t num_workers, const int32_t* schedule) {
  if (!context_lens) return fail(PMQA_ERR_INVALID_ARGUMENT, "context_lens is null");
  if (!schedule) return fail(PMQA_ERR_INVALID_ARGUMENT, "schedule is null");
  if (!aligned(context_lens, 4) || !aligned(schedule, 4))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "context_lens and schedule must be 4-byte aligned");
  if (batch < 1) return fail(PMQA_ERR_INVALID_ARGUMENT, "batch = %d must be >= 1", batch);
  if (num_workers < 1)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "num_workers = %d must be >= 1", num_workers);
  if (sched_words(batch, num_workers) > INT32_MAX)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "batch + 2*num_workers too large");
  return check_device(nullptr);
}

pmqa_status_t schedule_common(const int32_t* context_lens, int32_t batch, int32_t num_workers,
                              int32_t* schedule, bool linear, hipStream_t stream) {
  const pmqa_status_t st = check_schedule_args(context_lens, batch, num_workers, schedule);
  if (st != PMQA_OK) return st;
  const hipError_t e =
      pmqa::launch_schedule(context_lens, batch, num_workers, schedule, linear, stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "schedule launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

namespace {

// Validate mode for the append calls: every slot below num_pages * 64 (or
// negative), and no slot written twice.
pmqa_status_t validate_slots(const int64_t* slots, int64_t n, int64_t num_pages,
                             hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
  if (cap != hipStreamCaptureStatusNone)
    return fail(PMQA_ERR_CAPTURING, "PMQA_VALIDATE_INPUTS is set but the stream is capturing");
  std::vector<int64_t> h((size_t)n);
  e = hipMemcpyAsync(h.data(), slots, (size_t)n * 8, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "validate copy: %s", hipGetErrorString(e));
  for (int64_t i = 0; i < n; ++i)
    if (h[i] >= num_pages * pmqa::kPage)
      return fail(PMQA_ERR_INVALID_VALUE, "slot_mapping[%lld] = %lld outside [0, %lld)",
                  (long long)i, (long long)h[i], (long long)(num_pages * pmqa::kPage));
  std::sort(h.begin(), h.end());
  for (size_t i = 1; i < h.size(); ++i)
    if (h[i] >= 0 && h[i] == h[i - 1])
      return fail(PMQA_ERR_INVALID_VALUE, "slot %lld appears twice in slot_mapping",
                  (long long)h[i]);
  return PMQA_OK;
}

pmqa_status_t append_common(int variant, const void* k, int32_t k_dtype, int64_t num_tokens,
                            int32_t head_dim, const int64_t* slot_mapping, void* kv_cache,
                            int64_t num_pages, hipStream_t stream) {
  if (num_tokens < 0)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "num_tokens = %lld must be >= 0",
                (long long)num_tokens);
  if (num_tokens > (int64_t)INT32_MAX * 4)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "num_tokens = %lld too large", (long long)num_tokens);
  if (k_dtype != pmqa::kDtypeF32 && k_dtype != pmqa::kDtypeBf16)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "k_dtype = %d is neither PMQA_DTYPE_F32 nor "
                "PMQA_DTYPE_BF16", k_dtype);
  if (head_dim != pmqa::kHeadDim)
    return fail(PMQA_ERR_UNSUPPORTED, "head_dim = %d (compiled: %d)", head_dim, pmqa::kHeadDim);
  if (num_pages < 1)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "num_pages = %lld must be >= 1",
                (long long)num_pages);
  if (!kv_cache) return fail(PMQA_ERR_INVALID_ARGUMENT, "kv_cache is null");
  if (!aligned(kv_cache, 16))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "kv_cache must be 16-byte aligned");
  if (num_tokens == 0) return ok();  // nothing to read or write
  if (!k) return fail(PMQA_ERR_INVALID_ARGUMENT, "k is null");
  if (!slot_mapping) return fail(PMQA_ERR_INVALID_ARGUMENT, "slot_mapping is null");
  if (!aligned(k, 16)) return fail(PMQA_ERR_INVALID_ARGUMENT, "k must be 16-byte aligned");
  if (!aligned(slot_mapping, 8))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "slot_mapping must be 8-byte aligned");
  pmqa_status_t st = check_device(nullptr);
  if (st != PMQA_OK) return st;
  if (validate_mode()) {
    st = validate_slots(slot_mapping, num_tokens, num_pages, stream);
    if (st != PMQA_OK) return st;
  }
  const hipError_t e = pmqa::launch_append(variant, k, k_dtype, num_tokens, slot_mapping,
                                           static_cast<uint8_t*>(kv_cache), num_pages, stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

pmqa_status_t quantize_append_fp8(const void* k, int32_t k_dtype, int64_t num_tokens,
                                  int32_t head_dim, const int64_t* slot_mapping, void* kv_cache,
                                  int64_t num_pages, hipStream_t stream) {
  return append_common(0, k, k_dtype, num_tokens, head_dim, slot_mapping, kv_cache, num_pages,
                       stream);
}

pmqa_status_t quantize_append_fp4(const void* k, int32_t k_dtype, int64_t num_tokens,
                                  int32_t head_dim, const int64_t* slot_mapping, void* kv_cache,
                                  int64_t num_pages, hipStream_t stream) {
  return append_common(1, k, k_dtype, num_tokens, head_dim, slot_mapping, kv_cache, num_pages,
                       stream);
}

pmqa_status_t compute_schedule(const int32_t* context_lens, int32_t batch, int32_t num_workers,
                               int32_t* schedule, hipStream_t stream) {
  return schedule_common(context_lens, batch, num_workers, schedule, false, stream);
}

pmqa_status_t compute_schedule_linear(const int32_t* context_lens, int32_t batch,
                                      int32_t num_workers, int32_t* schedule,
                                      hipStream_t stream) {
  return schedule_common(context_lens, batch, num_workers, schedule, true, stream);
}

pmqa_status_t refresh_schedule(const int32_t* context_lens, int32_t batch, int32_t num_workers,
                               int32_t* schedule, int32_t* recomputed, hipStream_t stream) {
  if (recomputed && !aligned(recomputed, 4))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "recomputed must be 4-byte aligned");
  const pmqa_status_t st = check_schedule_args(context_lens, batch, num_workers, schedule);
  if (st != PMQA_OK) return st;
  const hipError_t e = pmqa::launch_refresh_schedule(context_lens, batch, num_workers, schedule,
                                                     recomputed, stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "refresh launch: %s", hipGetErrorString(e));
  return ok();
}

pmqa_status_t paged_mqa_logits_fp8(const void* q, const void* kv_cache, const float* weights,
                                   const int32_t* context_lens, const int32_t* block_table,
                                   const int32_t* schedule, float* logits, int32_t batch,
                                   int32_t next_n, int32_t num_heads, int32_t head_dim,
                                   int32_t page_size, int64_t num_pages,
                                   int32_t block_table_stride, int32_t max_context_len,
                                   int64_t logits_stride, int32_t num_workers,
                                   hipStream_t stream) {
  const Shape s{batch, next_n, block_table_stride, max_context_len, num_workers, num_pages,
                logits_stride};
  return logits_common(PMQA_VARIANT_FP8, q, nullptr, kv_cache, weights, context_lens,
                       block_table, schedule, logits, s, num_heads, head_dim, page_size, stream);
}

pmqa_status_t paged_mqa_logits_fp4(const void* q, const void* q_scale, const void* kv_cache,
                                   const float* weights, const int32_t* context_lens,
                                   const int32_t* block_table, const int32_t* schedule,
                                   float* logits, int32_t batch, int32_t next_n,
                                   int32_t num_heads, int32_t head_dim, int32_t page_size,
                                   int64_t num_pages, int32_t block_table_stride,
                                   int32_t max_context_len, int64_t logits_stride,
                                   int32_t num_workers, hipStream_t stream) {
  const Shape s{batch, next_n, block_table_stride, max_context_len, num_workers, num_pages,
                logits_stride};
  return logits_common(PMQA_VARIANT_FP4, q, q_scale, kv_cache, weights, context_lens,
                       block_table, schedule, logits, s, num_heads, head_dim, page_size, stream);
}

namespace {

pmqa_status_t check_topk_out(int32_t k, const int32_t* idx, const float* val, int64_t ldk,
                             int32_t rows, int32_t max_ctx, const void* ws, size_t ws_bytes) {
  if (k < 1) return fail(PMQA_ERR_INVALID_ARGUMENT, "k = %d must be >= 1", k);
  if (!idx) return fail(PMQA_ERR_INVALID_ARGUMENT, "topk_indices is null");
  if (!aligned(idx, 4) || (val && !aligned(val, 4)))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "topk_indices and topk_values must be 4-byte aligned");
  if (ldk < k)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "topk_stride = %lld must be >= k = %d",
                (long long)ldk, k);
  if (ws) {
    if (!aligned(ws, 16))
      return fail(PMQA_ERR_INVALID_ARGUMENT, "select_workspace must be 16-byte aligned");
    const size_t need = pmqa::select_workspace_bytes(rows, max_ctx, k);
    if (ws_bytes < need)
      return fail(PMQA_ERR_INVALID_ARGUMENT,
                  "select_workspace_bytes = %zu < %zu needed for %d rows", ws_bytes, need, rows);
  }
  return PMQA_OK;
}

pmqa_status_t topk_common(int variant, const void* q, const void* q_scale, const void* kv,
                          const float* weights, const int32_t* ctx, const int32_t* bt,
                          const int32_t* sched, float* workspace, int32_t k, int32_t* idx,
                          float* val, int64_t ldk, void* sel_ws, size_t sel_ws_bytes,
                          const Shape& s, int32_t num_heads, int32_t head_dim, int32_t page_size,
                          hipStream_t stream) {
  const int32_t rows = (int32_t)std::min<int64_t>((int64_t)s.batch * s.next_n, INT32_MAX);
  pmqa_status_t st = check_topk_out(k, idx, val, ldk, rows, s.max_ctx, sel_ws, sel_ws_bytes);
  if (st != PMQA_OK) return st;
  st = logits_common(variant, q, q_scale, kv, weights, ctx, bt, sched, workspace, s, num_heads,
                     head_dim, page_size, stream, /*fill=*/false);
  if (st != PMQA_OK) return st;
  int dev = 0;
  st = check_device(&dev);
  if (st != PMQA_OK) return st;
  const hipError_t e = pmqa::launch_select_topk(
      workspace, s.ldo, s.batch * s.next_n, s.max_ctx, nullptr, ctx, sched, s.batch, s.next_n,
      s.workers, k, idx, val, ldk, sel_ws, g_cus[dev].load(std::memory_order_acquire), stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "top-k launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

size_t pmqa_select_workspace_bytes(int32_t rows, int32_t max_context_len, int32_t k) {
  return pmqa::select_workspace_bytes(rows, max_context_len, k);
}

pmqa_status_t select_topk(const float* logits, int64_t logits_stride, int32_t rows,
                          int32_t max_context_len, const int32_t* lengths, int32_t k,
                          int32_t* topk_indices, float* topk_values, int64_t topk_stride,
                          void* select_workspace, size_t select_workspace_bytes,
                          hipStream_t stream) {
  if (!logits) return fail(PMQA_ERR_INVALID_ARGUMENT, "logits is null");
  if (!lengths) return fail(PMQA_ERR_INVALID_ARGUMENT, "lengths is null");
  if (!aligned(logits, 16))
    return fail(PMQA_ERR_INVALID_ARGUMENT, "logits must be 16-byte aligned");
  if (!aligned(lengths, 4)) return fail(PMQA_ERR_INVALID_ARGUMENT, "lengths must be 4-byte aligned");
  if (rows < 1) return fail(PMQA_ERR_INVALID_ARGUMENT, "rows = %d must be >= 1", rows);
  if (max_context_len < 1)
    return fail(PMQA_ERR_INVALID_ARGUMENT, "max_context_len = %d must be >= 1", max_context_len);
  if (logits_stride < max_context_len || logits_stride % 4 != 0)
    return fail(PMQA_ERR_INVALID_ARGUMENT,
                "logits_stride = %lld must be >= max_context_len and a multiple of 4",
                (long long)logits_stride);
  pmqa_status_t st = check_topk_out(k, topk_indices, topk_values, topk_stride, rows,
                                    max_context_len, select_workspace, select_workspace_bytes);
  if (st != PMQA_OK) return st;
  int dev = 0;
  st = check_device(&dev);
  if (st != PMQA_OK) return st;
  const hipError_t e = pmqa::launch_select_topk(
      logits, logits_stride, rows, max_context_len, lengths, nullptr, nullptr, 0, 1, 0, k,
      topk_indices, topk_values, topk_stride, select_workspace,
      g_cus[dev].load(std::memory_order_acquire), stream);
  if (e != hipSuccess) return fail(PMQA_ERR_HIP, "top-k launch: %s", hipGetErrorString(e));
  return ok();
}

pmqa_status_t select_topk_noalloc(const float* logits, int64_t logits_stride, int32_t rows,
                                  int32_t max_context_len, const int32_t* lengths, int32_t k,
                                  int32_t* topk_indices, float* topk_values,
                                  int64_t topk_stride, hipStream_t stream) {
  int dev = 0;
  pmqa_status_t st = check_device(&dev);
  if (st != PMQA_OK) return st;
  void* scratch = nullptr;
  const hipError_t e = pmqa::static_scratch(dev, &scratch);
  if (e != hipSuccess)
    return fail(PMQA_ERR_HIP, "static scratch of device %d: %s", dev, hipGetErrorString(e));
  const size_t need = pmqa::select_workspace_bytes(rows, max_context_len, k);
  const size_t have = pmqa::static_scratch_bytes();
  if (need > have)
    return fail(PMQA_ERR_INVALID_ARGUMENT,
                "%d rows of %d candidates with k = %d need %zu bytes of scratch; the static "
                "scratch holds %zu",
                rows, max_context_len, k, need, have);
  return select_topk(logits, logits_stride, rows, max_context_len, lengths, k, topk_indices,
                     topk_values, topk_stride, scratch, have, stream);
}

pmqa_status_t paged_mqa_topk_fp8(const void* q, const void* kv_cache, const float* weights,
                                 const int32_t* context_lens, const int32_t* block_table,
                                 const int32_t* schedule, float* logits_workspace, int32_t k,
                                 int32_t* topk_indices, float* topk_values, int64_t topk_stride,
                                 void* select_workspace, size_t select_workspace_bytes,
                                 int32_t batch, int32_t next_n, int32_t num_heads,
                                 int32_t head_dim, int32_t page_size, int64_t num_pages,
                                 int32_t block_table_stride, int32_t max_context_len,
                                 int64_t logits_stride, int32_t num_workers, hipStream_t stream) {
  const Shape s{batch, next_n, block_table_stride, max_context_len, num_workers, num_pages,
                logits_stride};
  return topk_common(PMQA_VARIANT_FP8, q, nullptr, kv_cache, weights, context_lens, block_table,
                     schedule, logits_workspace, k, topk_indices, topk_values, topk_stride,
                     select_workspace, select_workspace_bytes, s, num_heads, head_dim, page_size,
                     stream);
}

pmqa_status_t paged_mqa_topk_fp4(const void* q, const void* q_scale, const void* kv_cache,
                                 const float* weights, const int32_t* context_lens,
                                 const int32_t* block_table, const int32_t* schedule,
                                 float* logits_workspace, int32_t k, int32_t* topk_indices,
                                 float* topk_values, int64_t topk_stride, void* select_workspace,
                                 size_t select_workspace_bytes, int32_t batch, int32_t next_n,
                                 int32_t num_heads, int32_t head_dim, int32_t page_size,
                                 int64_t num_pages, int32_t block_table_stride,
                                 int32_t max_context_len, int64_t logits_stride,
                                 int32_t num_workers, hipStream_t stream) {
  const Shape s{batch, next_n, block_table_stride, max_context_len, num_workers, num_pages,
                logits_stride};
  return topk_common(PMQA_VARIANT_FP4, q, q_scale, kv_cache, weights, context_lens, block_table,
                     schedule, logits_workspace, k, topk_indices, topk_values, topk_stride,
                     select_workspace, select_workspace_bytes, s, num_heads, head_dim, page_size,
                     stream);
}

}  // extern "C"
