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
//   2. a block-wide exclusive scan of the slice sums (shuffles within each
//      wavefront, then the 16 wavefront totals) gives each slice's base; the
//      threads write the row prefix sums S[0..B] to the schedule buffer and,
//      for up to 12288 rows, to LDS;
//   3. after a barrier every worker w = 0..W takes g = floor(w*T/W) and finds
//      its row as upper_bound(S, g) - 1 (in LDS when the prefix sums fit
//      there), which can never land on a row with zero units
//      (S[b] <= g < S[b+1] implies c_b > 0).  The search is a binary search;
//      the linear scan it replaced (the "before" of the same section) is
//      kept as a second kernel with the identical result, to measure the
//      launch cost the change saves.
//
// The general lessons give the reuse rule: a schedule may be reused while no
// ceil(ctx_b / 256) has changed.  refresh_schedule_kernel is that rule on the
// device: it rebuilds the buffer only when the header does not describe this
// call or some row's unit count differs from the current lengths, so a graph
// that replays it on every step rewrites the schedule only when a row has
// crossed a 256-token boundary.
#include <hip/hip_runtime.h>

#include "pmqa_internal.h"

namespace pmqa {

namespace {

constexpr int kSchedThreads = 1024;
constexpr int kWaves = kSchedThreads / 64;
constexpr int kLdsPrefix = 12288;  // rows whose prefix sums are searched in LDS

__device__ inline int32_t units_of_len(int32_t len) {
  return len > 0 ? (int32_t)(((int64_t)len + kUnit - 1) / kUnit) : 0;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ inline int64_t wave_inclusive_scan(int64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// First index i in [0, n) with P[i] > g (n if none); P is non-decreasing.
template <class T>
__device__ inline int32_t upper_bound(const T* P, int32_t n, int64_t g) {
  int32_t a = 0;
  while (n > 0) {
    const int32_t half = n >> 1;
    if ((int64_t)P[a + half] <= g) {
      a += half + 1;
      n -= half + 1;
    } else {
      n = half;
    }
  }
  return a;
}

// The same index found by scanning P from the start.
template <class T>
__device__ inline int32_t upper_bound_linear(const T* P, int32_t n, int64_t g) {
  int32_t a = 0;
  while (a < n && (int64_t)P[a] <= g) ++a;
  return a;
}

struct SchedLds {
  int64_t wave_sums[kWaves];
  int32_t S[kLdsPrefix + 1];
};

// Writes the whole schedule (steps 1-3 above); every thread of the block
// calls it.
template <bool kLinear>
__device__ inline void build_schedule(const int32_t* __restrict__ ctx, int32_t batch,
                                      int32_t workers, int32_t* __restrict__ sched,
                                      SchedLds& lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int32_t* starts = sched + kSchedHeader;
  int32_t* S = starts + 2 * (workers + 1);
  int32_t* Sl = lds.S;
  const bool in_lds = batch <= kLdsPrefix;

  // 1. Each thread owns a contiguous slice of rows; sum their unit counts.
  const int32_t chunk = (batch + kSchedThreads - 1) / kSchedThreads;
  const int32_t lo = min(batch, tid * chunk);
  const int32_t hi = min(batch, lo + chunk);
  int64_t local = 0;
  for (int32_t b = lo; b < hi; ++b) local += units_of_len(ctx[b]);

  // 2. Block-wide exclusive scan: within each wave, then across waves.
  const int64_t incl = wave_inclusive_scan(local);
  if (lane == 63) lds.wave_sums[wave] = incl;
  __syncthreads();
  int64_t wave_base = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int64_t v = lds.wave_sums[w];
    wave_base += w < wave ? v : 0;
    total += v;
  }
  const bool fits = total <= (int64_t)INT32_MAX;
  int64_t run = wave_base + incl - local;
  for (int32_t b = lo; b < hi; ++b) {
    S[b] = (int32_t)run;
    if (in_lds) Sl[b] = (int32_t)run;
    run += units_of_len(ctx[b]);
  }
  if (tid == 0) {
    S[batch] = (int32_t)total;
    if (in_lds) Sl[batch] = (int32_t)total;
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

  // 3. Worker w starts at global unit floor(w*T/W): its row is the last b
  //    with S[b] <= g (never a row without units).
  for (int32_t w = tid; w <= workers; w += kSchedThreads) {
    int32_t row = batch, unit = 0;
    if (fits && w < workers) {
      const int64_t g = ((int64_t)w * total) / workers;
      int32_t a;
      if (kLinear)
        a = in_lds ? upper_bound_linear(Sl, batch + 1, g) : upper_bound_linear(S, batch + 1, g);
      else
        a = in_lds ? upper_bound(Sl, batch + 1, g) : upper_bound(S, batch + 1, g);
      row = a - 1;
      if (row >= batch) {  // g == total: nothing left for this worker
        row = batch;
        unit = 0;
      } else {
        unit = (int32_t)(g - (in_lds ? Sl[row] : S[row]));
      }
    }
    starts[2 * w] = row;
    starts[2 * w + 1] = unit;
  }
}

template <bool kLinear>
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ ctx,
                                                                 int32_t batch, int32_t workers,
                                                                 int32_t* __restrict__ sched) {
  __shared__ SchedLds lds;
  build_schedule<kLinear>(ctx, batch, workers, sched, lds);
}

// Leaves the buffer untouched when it already holds this call's schedule:
// header (magic, batch, workers, T) as compute_schedule writes it, S[0] = 0
// and S[b+1] - S[b] = ceil(ctx_b / 256) for every row (then S, T and the
// worker starts are what a rebuild would write).  Otherwise rebuilds it.
// *recomputed (when not null) receives 1 after a rebuild, else 0.
__global__ __launch_bounds__(kSchedThreads) void refresh_schedule_kernel(
    const int32_t* __restrict__ ctx, int32_t batch, int32_t workers, int32_t* __restrict__ sched,
    int32_t* __restrict__ recomputed) {
  __shared__ SchedLds lds;
  const int tid = threadIdx.x;
  const int32_t* S = sched + kSchedHeader + 2 * (workers + 1);
  bool fresh = sched[0] == kSchedMagic && sched[1] == batch && sched[2] == workers &&
               sched[4] == kUnit;
  if (fresh) {
    const int32_t chunk = (batch + kSchedThreads - 1) / kSchedThreads;
    const int32_t lo = min(batch, tid * chunk);
    const int32_t hi = min(batch, lo + chunk);
    for (int32_t b = lo; b < hi && fresh; ++b)
      fresh = S[b + 1] - S[b] == units_of_len(ctx[b]);
    if (tid == 0) fresh = fresh && S[0] == 0 && sched[3] == S[batch];
  }
  // Every read of the old contents happens before this barrier; a rebuild
  // only writes after it.
  fresh = __syncthreads_and(fresh);
  if (!fresh) build_schedule<false>(ctx, batch, workers, sched, lds);
  if (tid == 0 && recomputed) *recomputed = fresh ? 0 : 1;
}

}  // namespace

hipError_t launch_schedule(const int32_t* ctx, int32_t batch, int32_t num_workers, int32_t* sched,
                           bool linear, hipStream_t stream) {
  if (linear)
    hipLaunchKernelGGL(schedule_kernel<true>, dim3(1), dim3(kSchedThreads), 0, stream, ctx, batch,
                       num_workers, sched);
  else
    hipLaunchKernelGGL(schedule_kernel<false>, dim3(1), dim3(kSchedThreads), 0, stream, ctx,
                       batch, num_workers, sched);
  return hipGetLastError();
}

hipError_t launch_refresh_schedule(const int32_t* ctx, int32_t batch, int32_t num_workers,
                                   int32_t* sched, int32_t* recomputed, hipStream_t stream) {
  hipLaunchKernelGGL(refresh_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, ctx, batch,
                     num_workers, sched, recomputed);
  return hipGetLastError();
}

}  // namespace pmqa
