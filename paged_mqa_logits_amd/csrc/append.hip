// Quantize new K tokens and write them into the paged cache.
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
// introduction: the logits kernels read a paged K cache in fp8 (E4M3 values
// with one fp32 scale per token) and in fp4 (MXFP4: E2M1 values with one
// E8M0 scale per 32 values).  The page does not say how the cache is
// written; this is its producer, with the plainest rules those formats
// support:
//   fp8:   scale = amax / 448 (fp32, rounded to nearest even); code = the
//          E4M3fn value nearest to x / scale (|x / scale| clamped to 448),
//          ties to the even code, the sign bit following the sign of
//          x / scale; an all-zero token gets scale 0 and zero codes.
//   MXFP4: per 32 values, exponent e = floor(log2 amax) - 2 clamped to
//          [-127, 127] (E8M0 byte e + 127, or 0 for an all-zero block);
//          code = the E2M1 magnitude nearest to |x| * 2^-e, ties to the even
//          code, saturating at 6, sign bit only on a non-zero magnitude.
//
// Sixteen lanes per token: lane s of a token's group holds values 8s..8s+7
// (one 16-byte load for bf16), the token's amax (fp8) or each 32-value
// block's amax (MXFP4, 4 lanes) comes from a butterfly over the group, and
// each lane stores its 8 codes, so a token's codes are one contiguous
// 128-byte (fp8) or 64-byte (fp4) write.  A wavefront takes 4 tokens at a
// time and kTokenRounds rounds of them, all loads issued before any
// arithmetic.  The rounding itself is gfx950's conversion instructions
// (E4M3fn and scaled E2M1, both to nearest even); the per-value IEEE
// division x / scale of the fp8 rule is what bounds the kernel.
#include <hip/hip_runtime.h>

#include "pmqa_internal.h"

namespace pmqa {

namespace {

constexpr int kAppendThreads = 256;
constexpr int kTokenRounds = 4;                        // token rounds per wavefront
constexpr int kTokensPerWave = 4 * kTokenRounds;        // 4 tokens of 16 lanes per round
constexpr int kTokensPerBlock = (kAppendThreads / 64) * kTokensPerWave;

typedef float v8f __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Values 8s..8s+7 of token i as fp32 (bf16 widens exactly).
__device__ __forceinline__ v8f load_eight(const void* k, int32_t dtype, int64_t i, int s) {
  v8f x;
  if (dtype == kDtypeBf16) {
    const v4u w = static_cast<const v4u*>(k)[i * (kHeadDim / 8) + s];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float4* p = static_cast<const float4*>(k) + i * (kHeadDim / 4) + 2 * s;
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  return x;
}

// Max over groups of `width` consecutive lanes (width a power of two <= 64).
__device__ __forceinline__ float group_max(float v, int width) {
  for (int off = 1; off < width; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float abs_max8(const v8f& x) {
  float m = fabsf(x[0]);
#pragma unroll
  for (int e = 1; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  return m;
}

template <bool kFp4>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    const void* __restrict__ k, int32_t dtype, int64_t n, const int64_t* __restrict__ slots,
    uint8_t* __restrict__ kv, int64_t num_pages) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, s = lane & 15;  // token of the round, lane within it
  const int64_t base = ((int64_t)blockIdx.x * (kAppendThreads / 64) + (threadIdx.x >> 6)) *
                       (int64_t)kTokensPerWave;
  int64_t slot[kTokenRounds];
  v8f x[kTokenRounds];
#pragma unroll
  for (int r = 0; r < kTokenRounds; ++r) {
    const int64_t i = base + 4 * r + g;
    slot[r] = -1;
    x[r] = v8f{};
    if (i < n) {
      slot[r] = slots[i];
      x[r] = load_eight(k, dtype, i, s);
    }
  }
#pragma unroll
  for (int r = 0; r < kTokenRounds; ++r) {
    // every lane of the wavefront takes part in the butterflies; lanes of a
    // token without a valid slot store nothing
    const bool live = slot[r] >= 0 && slot[r] / kPage < num_pages;
    const v8f v = live ? x[r] : v8f{};
    const int64_t pg = live ? slot[r] / kPage : 0;
    const int row = live ? (int)(slot[r] % kPage) : 0;
    if (!kFp4) {
      const float amax = group_max(abs_max8(v), 16);
      const float scale = amax / 448.0f;
      uint32_t lo = 0, hi = 0;
      if (amax > 0.0f) {
        float q[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = fminf(fmaxf(v[e] / scale, -448.0f), 448.0f);
        // v_cvt_pk_fp8_f32 rounds to the nearest E4M3fn value, ties to
        // even, subnormals included, keeping the sign (|q| <= 448 here)
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)lo, true);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], (int)hi, true);
      }
      if (live) {
        uint8_t* page = kv + pg * (int64_t)kFp8PageBytes;
        reinterpret_cast<uint2*>(page + row * kHeadDim)[s] = make_uint2(lo, hi);
        if (s == 0) reinterpret_cast<float*>(page + kPage * kHeadDim)[row] = scale;
      }
    } else {
      // 32-value block = 4 lanes
      const float amax = group_max(abs_max8(v), 4);
      // floor(log2 amax) from the exponent field (an fp32-subnormal amax
      // has floor(log2) <= -127, which the clamp maps to the same e as
      // field 0)
      const int e = min(max((int)(__float_as_uint(amax) >> 23) - 127 - 2, -127), 127);
      uint32_t packed = 0, sbyte = 0;
      if (amax > 0.0f) {
        // v_cvt_scalef32_pk_fp4_f32 divides by the scale 2^e (exact) and
        // rounds to the nearest E2M1 value, ties to even, saturating at 6;
        // value 2i lands in the low nibble of byte i
        const float sc = __builtin_ldexpf(1.0f, e);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], sc, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], sc, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], sc, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], sc, 3);
        // a zero magnitude is stored without its sign bit
        const uint32_t m = packed & 0x77777777u;
        const uint32_t nz = (m | (m >> 1) | (m >> 2)) & 0x11111111u;
        packed = m | (packed & (nz << 3));
        sbyte = (uint32_t)(e + 127);
      }
      if (live) {
        uint8_t* page = kv + pg * (int64_t)kFp4PageBytes;
        reinterpret_cast<uint32_t*>(page + row * (kHeadDim / 2))[s] = packed;
        if ((s & 3) == 0) page[kPage * kHeadDim / 2 + row * (kHeadDim / 32) + s / 4] = sbyte;
      }
    }
  }
}

}  // namespace

hipError_t launch_append(int variant, const void* k, int32_t dtype, int64_t n,
                         const int64_t* slots, uint8_t* kv, int64_t num_pages,
                         hipStream_t stream) {
  const int64_t blocks = (n + kTokensPerBlock - 1) / kTokensPerBlock;
  if (variant == 0)
    hipLaunchKernelGGL(append_kernel<false>, dim3((uint32_t)blocks), dim3(kAppendThreads), 0,
                       stream, k, dtype, n, slots, kv, num_pages);
  else
    hipLaunchKernelGGL(append_kernel<true>, dim3((uint32_t)blocks), dim3(kAppendThreads), 0,
                       stream, k, dtype, n, slots, kv, num_pages);
  return hipGetLastError();
}

}  // namespace pmqa
