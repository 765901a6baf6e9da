// MXFP4 (E2M1 + E8M0 per 32 elements) instantiation of the persistent paged
// MQA logits kernel (page "[flashinfer] ... Paged MQA Logits ...",
// introduction: the fp4 kernel).
#include "logits_kernel.hpp"

namespace pmqa {

hipError_t launch_logits_fp4(const LogitsArgs& a, int next_n, int heads, hipStream_t stream) {
  return launch_logits<Fp4Format>(a, next_n, heads, stream);
}

hipError_t logits_blocks_per_cu(int variant, int next_n, int heads, int* blocks) {
  return variant == 0 ? blocks_per_cu<Fp8Format>(next_n, heads, blocks)
                      : blocks_per_cu<Fp4Format>(next_n, heads, blocks);
}

}  // namespace pmqa
