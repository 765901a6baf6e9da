// Internal host-side declarations shared by the C-ABI layer (api.cpp) and the
// HIP translation units that own the kernels.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace pmqa {

constexpr int kHeads = 64;  // the most heads a query row may have (also 32 or 16)
constexpr int kHeadDim = 128;
constexpr int kPage = 64;
constexpr int kUnit = 256;
constexpr int kPagesPerUnit = kUnit / kPage;
constexpr int kFp8PageBytes = kPage * kHeadDim + 4 * kPage;       // 8448
constexpr int kFp4PageBytes = kPage * kHeadDim / 2 + kPage * kHeadDim / 32;  // 4352
constexpr int kSchedHeader = 8;
constexpr int32_t kSchedMagic = 0x41514D50;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = 64 * kWavesPerBlock;

// Arguments of one logits launch (passed by value to the kernel).
struct LogitsArgs {
  const uint8_t* q;         // fp8: e4m3 [B, NN, H, D]; fp4: packed e2m1 [B, NN, H, D/2]
  const uint8_t* q_scale;   // fp4 only: e8m0 [B, NN, H, D/32]
  const uint8_t* kv;        // [num_pages][page bytes]
  const float* weights;     // [B*NN, H]
  const int32_t* ctx;       // [B]
  const int32_t* bt;        // [B, bt_stride]
  const int32_t* sched;     // compute_schedule output
  float* out;               // [B*NN, ldo]
  int64_t num_pages;
  int64_t ldo;
  int32_t batch;
  int32_t bt_stride;
  int32_t max_ctx;
  int32_t num_workers;
  uint32_t flush_ticks;     // period of the synchronised stage flushes (set by the launcher)
  int32_t fill_tails;       // 1: the unit kernel also writes -inf past every row's units
};

// Launchers (defined next to their kernels).  Return the launch status.
// linear: find worker starts by a linear scan instead of a binary search
// (same result).
hipError_t launch_schedule(const int32_t* ctx, int32_t batch, int32_t num_workers,
                           int32_t* sched, bool linear, hipStream_t stream);
// Rebuilds sched only when it does not match (batch, num_workers, ctx).
hipError_t launch_refresh_schedule(const int32_t* ctx, int32_t batch, int32_t num_workers,
                                   int32_t* sched, int32_t* recomputed, hipStream_t stream);
// heads: 64, 32 or 16.
hipError_t launch_logits_fp8(const LogitsArgs& a, int next_n, int heads, hipStream_t stream);
hipError_t launch_logits_fp4(const LogitsArgs& a, int next_n, int heads, hipStream_t stream);
// -inf over columns [0, max_ctx) of every output row (runs before the unit
// kernel, which overwrites the scheduled units).
hipError_t launch_neg_inf_fill(float* out, int64_t ldo, int64_t rows, int32_t max_ctx,
                               int32_t blocks, hipStream_t stream);

// Element types of the K values handed to the append kernels.
constexpr int32_t kDtypeF32 = 0;
constexpr int32_t kDtypeBf16 = 1;
// Quantize n tokens of K [n, 128] (fp32 or bf16) into the paged cache at
// slots[i] = page * 64 + row; negative slots and pages >= num_pages are
// skipped.  variant 0 = fp8 pages, 1 = MXFP4 pages.
hipError_t launch_append(int variant, const void* k, int32_t dtype, int64_t n,
                         const int64_t* slots, uint8_t* kv, int64_t num_pages,
                         hipStream_t stream);

// Top-k per row of logits [rows, ldo]: candidates are the first
// lengths[r] columns (lengths given), else the fused indexer rule from
// ctx / sched (batch, next_n, workers).  Writes out_idx [rows, ldk] and,
// when not null, out_val [rows, ldk].  workspace: null, or at least
// select_workspace_bytes(rows, max_ctx, k) bytes, 16-byte aligned (unused
// when that is 0); with it, long rows are split over several workgroups.
// cus: compute units of the device.
constexpr int32_t kSplitRows = 512;  // two rows per compute unit of an MI355X
size_t select_workspace_bytes(int32_t rows, int32_t max_ctx, int32_t k);
// The allocation-free selection's scratch: a static device array of
// static_scratch_bytes() bytes (enough for select_workspace_bytes of any
// call); static_scratch(dev, &p) gives device dev's copy, looked up once per
// device.
size_t static_scratch_bytes();
hipError_t static_scratch(int dev, void** ptr);
hipError_t launch_select_topk(const float* logits, int64_t ldo, int32_t rows, int32_t max_ctx,
                              const int32_t* lengths, const int32_t* ctx, const int32_t* sched,
                              int32_t batch, int32_t next_n, int32_t workers, int32_t k,
                              int32_t* out_idx, float* out_val, int64_t ldk, void* workspace,
                              int32_t cus, hipStream_t stream);

// Resident workgroups per compute unit of a logits kernel (occupancy query).
hipError_t logits_blocks_per_cu(int variant, int next_n, int heads, int* blocks);

}  // namespace pmqa
