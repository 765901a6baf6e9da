// -inf fill of the logits region, run before the unit kernel (for outputs
// above 32 MB; smaller ones are filled past their units by the unit
// kernel's own workers).
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
// introduction: positions past a row's context carry no score; they are -inf
// in the output.  This kernel writes -inf over every column [0, M) of every
// output row; the unit kernel that runs after it on the same stream then
// overwrites the columns of each scheduled 256-token unit (scores, or -inf
// past the causal limit).  The final output therefore never depends on which
// units the schedule holds: every column not covered by a unit stays -inf.
//
// Filling the whole region costs ~9% more bytes than filling only the
// columns past each row's last unit, but measured on MI355X it is faster: a
// branch-free sweep keeps HBM writes dense.  The sweep: thread i of the grid
// writes 16-byte quads i, i + G, ... of the row-major [rows, M] region (G =
// grid threads), so at any moment the grid writes G consecutive quads (one
// workgroup per compute unit for strided rows; for contiguous rows, below,
// fewer writers with four quads in flight each).  Stores are non-temporal:
// plain stores leave dirty L2 lines whose write-back then competes with the
// next kernel's reads.
#include <hip/hip_runtime.h>

#include "pmqa_internal.h"

namespace pmqa {

namespace {

constexpr int kFillThreads = 256;

typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kFillThreads) void neg_inf_fill_kernel(float* __restrict__ out,
                                                                    int64_t ldo, int64_t rows,
                                                                    int32_t max_ctx) {
  const uint32_t quads = (uint32_t)(max_ctx + 3) / 4;  // per row
  const uint32_t stride = gridDim.x * kFillThreads;
  const uint32_t first = blockIdx.x * kFillThreads + threadIdx.x;
  const uint32_t dr = stride / quads, dq = stride - dr * quads;
  int64_t r = first / quads;
  uint32_t q = first - (uint32_t)r * quads;
  const float ninf = -__builtin_inff();
  const v4f nv = {ninf, ninf, ninf, ninf};
  while (r < rows) {
    const int32_t col = (int32_t)(4 * q);
    float* dst = out + r * ldo + col;
    if (col + 4 <= max_ctx) {
      __builtin_nontemporal_store(nv, reinterpret_cast<v4f*>(dst));
    } else {
      for (int e = 0; e < 4; ++e)
        if (col + e < max_ctx) dst[e] = ninf;
    }
    q += dq;
    r += dr;
    if (q >= quads) {
      q -= quads;
      ++r;
    }
  }
}

// The same sweep over a region whose rows are contiguous (ldo == max_ctx, a
// multiple of 4): one flat range of quads, with no row arithmetic per store.
// Fewer writers with more stores each write faster here: measured on
// MI355X over 537 MB, one workgroup of 128 threads per four compute units,
// each thread storing 4 quads a grid stride apart per round, sweeps in 74 us
// (7.2 TB/s); one workgroup of 256 threads per compute unit, one quad per
// round, in 84 us (6.4 TB/s); more threads or workgroups are slower still.
constexpr int kFlatThreads = 128;
constexpr int kFlatUnroll = 4;

__global__ __launch_bounds__(kFlatThreads) void neg_inf_fill_flat_kernel(v4f* __restrict__ out,
                                                                         int64_t quads) {
  const float ninf = -__builtin_inff();
  const v4f nv = {ninf, ninf, ninf, ninf};
  const int64_t stride = (int64_t)gridDim.x * kFlatThreads;
  int64_t i = (int64_t)blockIdx.x * kFlatThreads + threadIdx.x;
  for (; i + (kFlatUnroll - 1) * stride < quads; i += kFlatUnroll * stride) {
#pragma unroll
    for (int u = 0; u < kFlatUnroll; ++u) __builtin_nontemporal_store(nv, out + i + u * stride);
  }
  for (; i < quads; i += stride) __builtin_nontemporal_store(nv, out + i);
}

}  // namespace

hipError_t launch_neg_inf_fill(float* out, int64_t ldo, int64_t rows, int32_t max_ctx,
                               int32_t blocks, hipStream_t stream) {
  if (ldo == max_ctx && max_ctx % 4 == 0)
    hipLaunchKernelGGL(neg_inf_fill_flat_kernel, dim3(blocks >= 8 ? blocks / 4 : 2),
                       dim3(kFlatThreads), 0, stream, reinterpret_cast<v4f*>(out),
                       rows * (int64_t)(max_ctx / 4));
  else
    hipLaunchKernelGGL(neg_inf_fill_kernel, dim3(blocks), dim3(kFillThreads), 0, stream, out,
                       ldo, rows, max_ctx);
  return hipGetLastError();
}

}  // namespace pmqa
