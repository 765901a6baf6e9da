/*
 * pmqa_ceiling.h - C ABI of the streaming ceiling kernels (libpmqa_ceiling.so),
 * a measurement library beside the paged MQA logits library.
 *
 * Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
 * section 1, first bullet: the Blackwell kernels move K pages with bulk
 * tensor-memory copies.  A paged MQA logits call on gfx950 reads the pages of
 * every scored token with 16-byte non-temporal buffer loads and writes an
 * output region of batch*next_n*max_context_len fp32 values.  These two
 * calls do only that data movement, with no arithmetic, so the rate they
 * reach on a device is the practical ceiling the logits call is compared to.
 *
 * Conventions: device pointers, caller-owned buffers, asynchronous on
 * `stream`, nothing allocated, no host synchronization.  Return value: 0 on
 * success, 1 for an invalid argument (nothing is launched), 2 when the launch
 * failed.
 */
#ifndef PMQA_CEILING_H
#define PMQA_CEILING_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PMQA_CEILING_FP8_PAGE_BYTES 8448 /* 64 tokens x 128 e4m3 + 64 fp32 scales */
#define PMQA_CEILING_FP4_PAGE_BYTES 4352 /* 64 tokens x 64 packed e2m1 + 64 x 4 e8m0 */
#define PMQA_CEILING_THREADS 256         /* threads per workgroup (one wavefront per SIMD) */

/*
 * pmqa_ceiling_gather - load every byte of n_pages pages of a paged K cache.
 *
 *   kv_cache         [num_pages][page_bytes] bytes, 16-byte aligned.
 *   page_bytes       PMQA_CEILING_FP8_PAGE_BYTES or PMQA_CEILING_FP4_PAGE_BYTES.
 *   pages            int32 [n_pages] page ids, 4-byte aligned; ids outside
 *                    [0, num_pages) are clamped into it.
 *   num_blocks       workgroups of PMQA_CEILING_THREADS threads; wavefront w
 *                    of the num_blocks*4 loads the contiguous share
 *                    [w*n_pages/W, (w+1)*n_pages/W) of the list, whole pages
 *                    of 1 KB per load instruction.  num_blocks = compute units
 *                    x k runs k wavefronts per SIMD.
 *   pages_in_flight  2 or 4: pages each wavefront keeps in flight.
 *   sink             num_blocks*PMQA_CEILING_THREADS*16 bytes, 16-byte aligned:
 *                    each thread stores the XOR of the 16-byte words it loaded
 *                    (so no load can be dropped); the value has no other use.
 */
int pmqa_ceiling_gather(const void* kv_cache, int64_t num_pages, int32_t page_bytes,
                        const int32_t* pages, int64_t n_pages, int32_t num_blocks,
                        int32_t pages_in_flight, void* sink, hipStream_t stream);

/*
 * pmqa_ceiling_fill - write `value` over n_floats consecutive fp32 values
 * with 16-byte non-temporal stores, a grid-stride sweep of num_blocks
 * workgroups of `threads` threads (64, 128 or 256), each thread storing
 * stores_per_round (1 or 4) quads a grid stride apart per round.
 *
 *   out       16-byte aligned; n_floats >= 4 and a multiple of 4.
 */
int pmqa_ceiling_fill(float* out, int64_t n_floats, float value, int32_t num_blocks,
                      int32_t threads, int32_t stores_per_round, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PMQA_CEILING_H */
