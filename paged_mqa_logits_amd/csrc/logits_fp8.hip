// fp8 (E4M3 + per-token fp32 scale) instantiation of the persistent paged
// MQA logits kernel (page "[flashinfer] ... Paged MQA Logits ...",
// introduction: the fp8 kernel).
#include "logits_kernel.hpp"

namespace pmqa {

hipError_t launch_logits_fp8(const LogitsArgs& a, int next_n, int heads, hipStream_t stream) {
  return launch_logits<Fp8Format>(a, next_n, heads, stream);
}

}  // namespace pmqa
