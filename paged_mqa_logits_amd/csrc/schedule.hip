// GPU-side persistent-worker schedule for paged MQA logits.
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
// sections 1-2: the per-call partition of work over persistent workers is
// computed on the GPU (no host round trip, so it can be graph-captured), and
// each worker's start is found by a binary search instead of a linear scan.
// The general lessons fix the work unit: 256 tokens of one row, so the result
// stays valid only while every ceil(context_len / 256) is unchanged.
//
// One workgroup of 1024 threads:
//   1. thread i owns a contiguous slice of rows and sums their unit counts
//      c_b = ceil(ctx_b / 256) (negative lengths count as 0);
//   2. a block-wide exclusive scan of the slice sums gives each slice's base;
//      the threads write the row prefix sums S[0..B] to the schedule buffer;
//   3. after a barrier every worker w = 0..W takes g = floor(w*T/W) and finds
//      its row as upper_bound(S, g) - 1 by binary search, which can never land
//      on a row with zero units (S[b] <= g < S[b+1] implies c_b > 0).
#include <hip/hip_runtime.h>

#include "pmqa_internal.h"

namespace pmqa {

namespace {

constexpr int kSchedThreads = 1024;

__device__ inline int32_t units_of_len(int32_t len) {
  return len > 0 ? (int32_t)(((int64_t)len + kUnit - 1) / kUnit) : 0;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ ctx,
                                                                 int32_t batch, int32_t workers,
                                                                 int32_t* __restrict__ sched) {
  __shared__ int64_t scan[kSchedThreads];
  const int tid = threadIdx.x;
  int32_t* starts = sched + kSchedHeader;
  int32_t* S = starts + 2 * (workers + 1);

  const int32_t chunk = (batch + kSchedThreads - 1) / kSchedThreads;
  const int32_t lo = min(batch, tid * chunk);
  const int32_t hi = min(batch, lo + chunk);
  int64_t local = 0;
  for (int32_t b = lo; b < hi; ++b) local += units_of_len(ctx[b]);

  // Hillis-Steele inclusive scan over the 1024 slice sums.
  scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    int64_t v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int64_t total = scan[kSchedThreads - 1];
  const bool fits = total <= (int64_t)INT32_MAX;

  int64_t run = scan[tid] - local;  // exclusive base of this slice
  for (int32_t b = lo; b < hi; ++b) {
    S[b] = (int32_t)run;
    run += units_of_len(ctx[b]);
  }
  if (tid == 0) {
    S[batch] = (int32_t)total;
    sched[0] = kSchedMagic;
    sched[1] = batch;
    sched[2] = workers;
    sched[3] = fits ? (int32_t)total : -1;
    sched[4] = kUnit;
    sched[5] = 0;
    sched[6] = 0;
    sched[7] = 0;
  }
  // Make the prefix sums written above visible to every thread of the block.
  __threadfence_block();
  __syncthreads();

  for (int32_t w = tid; w <= workers; w += kSchedThreads) {
    int32_t row = batch, unit = 0;
    if (fits && w < workers) {
      const int64_t g = ((int64_t)w * total) / workers;
      // first index i in [0, batch] with S[i] > g
      int32_t a = 0, n = batch + 1;
      while (n > 0) {
        const int32_t half = n >> 1;
        if ((int64_t)S[a + half] <= g) {
          a += half + 1;
          n -= half + 1;
        } else {
          n = half;
        }
      }
      row = a - 1;
      if (row >= batch) {  // g == total: nothing left for this worker
        row = batch;
        unit = 0;
      } else {
        unit = (int32_t)(g - S[row]);
      }
    }
    starts[2 * w] = row;
    starts[2 * w + 1] = unit;
  }
}

}  // namespace

hipError_t launch_schedule(const int32_t* ctx, int32_t batch, int32_t num_workers, int32_t* sched,
                           hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, ctx, batch,
                     num_workers, sched);
  return hipGetLastError();
}

}  // namespace pmqa
