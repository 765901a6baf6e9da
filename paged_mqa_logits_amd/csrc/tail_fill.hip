// -inf fill of the logits columns that no work unit covers.
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
// introduction: positions past a row's context carry no score; they are -inf
// in the output.  The unit kernel writes every column of every scheduled
// 256-token unit (scores, or -inf past the causal limit); this kernel writes
// -inf over the rest of each row, columns [min(256 * c_b, M), M), where c_b is
// the row's unit count in the same schedule, so together they write every
// column in [0, M) exactly once.  A schedule whose header does not match the
// call is not used by either kernel, and this kernel then fills every column.
//
// HBM writes run fastest when the whole GPU sweeps a compact window of
// addresses: one workgroup per compute unit, and thread i of the grid writes
// 16-byte quads i, i + G, i + 2G, ... of the row-major [rows, M] region
// (G = grid threads), so at any moment the grid writes G consecutive quads.
// Each workgroup first caches every row's first -inf column in LDS, so the
// sweep itself issues nothing but stores.
// The kernel runs after the unit kernel: writing this 90%-of-the-output
// region last keeps its write-back traffic out of the read-heavy phase.
#include <hip/hip_runtime.h>

#include "pmqa_internal.h"

namespace pmqa {

namespace {

constexpr int kFillThreads = 256;
constexpr int kLdsRows = 16384;  // rows whose tail start is cached in LDS

typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int32_t tail_start(const int32_t* S, bool ok, int64_t r, int32_t next_n,
                                              int32_t cap, int32_t max_ctx) {
  const int32_t b = (int32_t)(r / next_n);
  const int32_t c = ok ? min(max(S[b + 1] - S[b], 0), cap) : 0;
  return min(c * kUnit, max_ctx);
}

__global__ __launch_bounds__(kFillThreads) void tail_fill_kernel(float* __restrict__ out, int64_t ldo,
                                                                 int32_t batch, int32_t next_n,
                                                                 int32_t max_ctx,
                                                                 const int32_t* __restrict__ sched,
                                                                 int32_t workers) {
  __shared__ int32_t ts_lds[kLdsRows];
  const bool ok = sched[0] == kSchedMagic && sched[1] == batch && sched[2] == workers &&
                  sched[3] >= 0;
  const int32_t* S = sched + kSchedHeader + 2 * (workers + 1);
  const int32_t cap = (max_ctx + kUnit - 1) / kUnit;
  const int64_t rows = (int64_t)batch * next_n;
  const bool cached = rows <= kLdsRows;
  if (cached) {
    for (int32_t r = threadIdx.x; r < rows; r += kFillThreads)
      ts_lds[r] = tail_start(S, ok, r, next_n, cap, max_ctx);
  }
  __syncthreads();
  // Thread i writes quads i, i + G, i + 2G, ... of the row-major region; the
  // stride G is split once into whole rows and a remainder.
  const uint32_t quads = (uint32_t)(max_ctx + 3) / 4;  // per row
  const uint32_t stride = gridDim.x * kFillThreads;
  const uint32_t first = blockIdx.x * kFillThreads + threadIdx.x;
  const uint32_t dr = stride / quads, dq = stride - dr * quads;
  int64_t r = first / quads;
  uint32_t q = first - (uint32_t)r * quads;
  const float ninf = -__builtin_inff();
  const v4f nv = {ninf, ninf, ninf, ninf};
  while (r < rows) {
    const int32_t ts = cached ? ts_lds[r] : tail_start(S, ok, r, next_n, cap, max_ctx);
    const int32_t col = (int32_t)(4 * q);
    if (col >= ts) {
      float* dst = out + r * ldo + col;
      if (col + 4 <= max_ctx) {
        __builtin_nontemporal_store(nv, reinterpret_cast<v4f*>(dst));
      } else {
        for (int e = 0; e < 4; ++e)
          if (col + e < max_ctx) dst[e] = ninf;
      }
    }
    q += dq;
    r += dr;
    if (q >= quads) {
      q -= quads;
      ++r;
    }
  }
}

}  // namespace

hipError_t launch_tail_fill(float* out, int64_t ldo, int32_t batch, int32_t next_n,
                            int32_t max_ctx, const int32_t* sched, int32_t workers, int32_t blocks,
                            hipStream_t stream) {
  hipLaunchKernelGGL(tail_fill_kernel, dim3(blocks), dim3(kFillThreads), 0, stream, out, ldo,
                     batch, next_n, max_ctx, sched, workers);
  return hipGetLastError();
}

}  // namespace pmqa
