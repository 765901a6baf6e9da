// Streaming ceiling kernels: the HBM rate MI355X reaches for the byte mix of
// a paged MQA logits call when nothing is computed.
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
// section 1, first bullet: the Blackwell kernels bring K pages in with bulk
// tensor-memory copies.  On gfx950 the logits kernel streams the same pages
// with 16-byte non-temporal buffer loads, and writes its output region
// (mostly -inf) with non-temporal stores.  The two kernels here do only that
// data movement, over the same pages and the same output size, so their rate
// is the practical ceiling of the call on the box it runs on:
//
//   ceiling_gather_kernel  every wavefront walks a contiguous share of a
//       list of page ids (the pages a call reads, in row order) and loads
//       each page whole, 1 KB per load instruction (64 lanes x 16 bytes),
//       with F pages in flight in a ring of registers; the loaded words are
//       folded with XOR into one register per lane, stored at the end so
//       the loads cannot be dropped.
//   ceiling_fill_kernel    a grid-stride sweep of 16-byte non-temporal
//       stores over a contiguous region: at any moment the grid writes one
//       window of consecutive quads.
//
// Both take their workgroup count from the caller, so a sweep over waves per
// SIMD (workgroups per compute unit) and pages in flight finds the best
// shape.  Measurement code only: the logits library does not use them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_ceiling.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;

constexpr int kThreads = 256;          // 4 wavefronts: one per SIMD of a compute unit
constexpr int kRsrcWord3 = 0x00020000; // raw buffer, 32-bit data format
constexpr int kLoadNT = 2;             // non-temporal load

__device__ __forceinline__ int32_t sload(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane(*(cint_ptr)(p));
}

__device__ __forceinline__ rsrc_t page_rsrc(const uint8_t* kv, int64_t pid, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kv + pid * bytes), 0,
                                           (int32_t)bytes, kRsrcWord3);
}

// L = loads per page (ceil(page_bytes / 1024)).  id is the page's entry of
// the list (read one iteration ahead); ok false: past the wave's share, a
// zero-size resource, so the loads return zeros without touching memory and
// every slot issues the same instructions.
template <int L>
__device__ __forceinline__ void load_page(const uint8_t* kv, int64_t num_pages, int32_t id,
                                          bool ok, uint32_t page_bytes, int lane,
                                          v4i (&slot)[L]) {
  const int64_t pid = id < 0 ? 0 : (id >= num_pages ? num_pages - 1 : id);
  const rsrc_t r = page_rsrc(kv, ok ? pid : 0, ok ? page_bytes : 0u);
#pragma unroll
  for (int i = 0; i < L; ++i)
    slot[i] = __builtin_amdgcn_raw_buffer_load_b128(r, 1024 * i + 16 * lane, 0, kLoadNT);
}

// F = pages in flight per wavefront.
template <int L, int F>
__global__ __launch_bounds__(kThreads) void ceiling_gather_kernel(
    const uint8_t* __restrict__ kv, int64_t num_pages, uint32_t page_bytes,
    const int32_t* __restrict__ pages, int64_t n_pages, v4i* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) +
                    __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t p0 = w * n_pages / waves, p1 = (w + 1) * n_pages / waves;
  const int64_t last = n_pages - 1;
  v4i acc = {0, 0, 0, 0};
  v4i ring[F][L];
  int32_t ids[F];  // list entries of the pages loaded next (p + F + f)
#pragma unroll
  for (int f = 0; f < F; ++f) {
    load_page<L>(kv, num_pages, sload(pages + min(p0 + f, last)), p0 + f < p1, page_bytes, lane,
                 ring[f]);
    ids[f] = sload(pages + min(p0 + F + f, last));
  }
  // One exit at the loop's end keeps the load counter's history the same on
  // every path, so consuming slot f waits only for its own page; the
  // scheduling barriers keep each slot's refill right after its use (left
  // alone, the compiler drains every slot before issuing any refill).
  for (int64_t p = p0;; p += F) {
    int32_t nids[F];
#pragma unroll
    for (int f = 0; f < F; ++f) nids[f] = sload(pages + min(p + 2 * F + f, last));
#pragma unroll
    for (int f = 0; f < F; ++f) {
#pragma unroll
      for (int i = 0; i < L; ++i) acc ^= ring[f][i];
      load_page<L>(kv, num_pages, ids[f], p + F + f < p1, page_bytes, lane, ring[f]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int f = 0; f < F; ++f) ids[f] = nids[f];
    if (p + F >= p1) break;
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// U = 16-byte stores per thread per round, a grid stride apart.
template <int U>
__global__ __launch_bounds__(kThreads) void ceiling_fill_kernel(v4f* __restrict__ out,
                                                                int64_t n_quads, float value) {
  const v4f v = {value, value, value, value};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (U - 1) * stride < n_quads; i += U * stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v, out + i + u * stride);
  }
  for (; i < n_quads; i += stride) __builtin_nontemporal_store(v, out + i);
}

template <int L>
hipError_t launch_gather(const uint8_t* kv, int64_t num_pages, uint32_t page_bytes,
                         const int32_t* pages, int64_t n_pages, int32_t blocks, int32_t in_flight,
                         v4i* sink, hipStream_t stream) {
  if (in_flight == 2)
    hipLaunchKernelGGL((ceiling_gather_kernel<L, 2>), dim3(blocks), dim3(kThreads), 0, stream,
                       kv, num_pages, page_bytes, pages, n_pages, sink);
  else
    hipLaunchKernelGGL((ceiling_gather_kernel<L, 4>), dim3(blocks), dim3(kThreads), 0, stream,
                       kv, num_pages, page_bytes, pages, n_pages, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" int pmqa_ceiling_gather(const void* kv_cache, int64_t num_pages, int32_t page_bytes,
                                   const int32_t* pages, int64_t n_pages, int32_t num_blocks,
                                   int32_t pages_in_flight, void* sink, hipStream_t stream) {
  if (!kv_cache || !pages || !sink || num_pages < 1 || n_pages < 1 || num_blocks < 1) return 1;
  if ((uintptr_t)kv_cache % 16 || (uintptr_t)sink % 16 || (uintptr_t)pages % 4) return 1;
  if (pages_in_flight != 2 && pages_in_flight != 4) return 1;
  const uint8_t* kv = static_cast<const uint8_t*>(kv_cache);
  v4i* out = static_cast<v4i*>(sink);
  hipError_t e;
  if (page_bytes == PMQA_CEILING_FP8_PAGE_BYTES)
    e = launch_gather<9>(kv, num_pages, (uint32_t)page_bytes, pages, n_pages, num_blocks,
                         pages_in_flight, out, stream);
  else if (page_bytes == PMQA_CEILING_FP4_PAGE_BYTES)
    e = launch_gather<5>(kv, num_pages, (uint32_t)page_bytes, pages, n_pages, num_blocks,
                         pages_in_flight, out, stream);
  else
    return 1;
  return e == hipSuccess ? 0 : 2;
}

extern "C" int pmqa_ceiling_fill(float* out, int64_t n_floats, float value, int32_t num_blocks,
                                 int32_t threads, int32_t stores_per_round, hipStream_t stream) {
  if (!out || n_floats < 4 || n_floats % 4 || num_blocks < 1 || (uintptr_t)out % 16) return 1;
  if ((threads != 64 && threads != 128 && threads != 256) ||
      (stores_per_round != 1 && stores_per_round != 4))
    return 1;
  if (stores_per_round == 1)
    hipLaunchKernelGGL(ceiling_fill_kernel<1>, dim3(num_blocks), dim3(threads), 0, stream,
                       reinterpret_cast<v4f*>(out), n_floats / 4, value);
  else
    hipLaunchKernelGGL(ceiling_fill_kernel<4>, dim3(num_blocks), dim3(threads), 0, stream,
                       reinterpret_cast<v4f*>(out), n_floats / 4, value);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
