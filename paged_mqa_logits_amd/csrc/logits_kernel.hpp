// Persistent paged MQA logits kernel for gfx950, shared by the fp8 and MXFP4
// element formats.
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입":
// introduction (per-head weighted sum of rectified scores, fp8 and fp4
// kernels), section 1 (the task iterator skips zero-length rows) and the
// general lessons (lookahead and the task iterator must pick the same rows).
//
// Mapping onto CDNA4
// ------------------
// One worker is one 64-lane wavefront.  A worker walks its schedule range of
// 256-token units page by page (64 tokens).  For a page it contracts the
// 64-head query block of each query row against the page's 64 K rows with
// v_mfma_scale_f32_16x16x128_f8f6f4: K = head_dim = 128 is covered by one
// instruction, so a page is 4 head groups x 4 token groups x next_n MFMAs.
//
//   A operand (query): lane l holds head 16*hg + (l & 15), elements
//     [32*(l>>4), +32) of head_dim.  Loaded once per batch row.
//   B operand (K):     lane l holds token 16*tg + (l & 15), the same element
//     range.  Loaded straight from HBM into VGPRs with 16-byte loads: every
//     K byte is used by exactly one lane, so no LDS staging is needed.
//   C (scores):        lane l holds heads 16*hg + 4*(l>>4) + i, i = 0..3, of
//     token 16*tg + (l & 15).
//
// Epilogue per (head, token): one v_med3 (ReLU, or its mirror for a negative
// token scale) and one FMA with the head weight; the 16 heads of a lane are
// summed in registers, then the four lane groups are reduced and scattered
// with permlane32/permlane16 swaps so that lane l ends up owning token l of
// the page and the 64 results are stored as one contiguous 256-byte row.
//
// Software pipeline: the K fragment of the next page is requested before the
// current page is contracted.  Both the lookahead and the consumer use the
// same iterator function, so they always agree on which (row, unit, page)
// comes next, including across skipped zero-length rows.
//
// After its units, every worker writes -inf over an equal share of the
// 256-column chunks that lie past each row's last unit (the tail fill), with
// 16-byte non-temporal stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_internal.h"

namespace pmqa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0;  // cbsz/blgp code of E4M3 operands
constexpr int kFmtFp4 = 4;  // cbsz/blgp code of E2M1 operands
constexpr int kScaleOne = 127;  // E8M0 encoding of 1.0

__device__ __forceinline__ int32_t sload(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane(*p);
}

// Read-only view of a schedule; every index derived from it is clamped.
struct SchedView {
  const int32_t* starts;
  const int32_t* S;
  int32_t rows;      // batch rows covered (0 when the schedule is unusable)
  int32_t cap;       // units per row never exceed ceil(max_ctx / 256)
};

__device__ __forceinline__ SchedView make_view(const LogitsArgs& a) {
  SchedView v;
  const int32_t magic = sload(a.sched + 0);
  const int32_t b = sload(a.sched + 1);
  const int32_t w = sload(a.sched + 2);
  const int32_t t = sload(a.sched + 3);
  const bool ok = magic == kSchedMagic && b == a.batch && w == a.num_workers && t >= 0;
  v.starts = a.sched + kSchedHeader;
  v.S = v.starts + 2 * (a.num_workers + 1);
  v.rows = ok ? a.batch : 0;
  v.cap = (a.max_ctx + kUnit - 1) / kUnit;
  return v;
}

__device__ __forceinline__ int32_t units_of(const SchedView& v, int32_t b) {
  const int32_t c = sload(v.S + b + 1) - sload(v.S + b);
  return min(max(c, 0), v.cap);
}

// One page of work: batch row b, unit u, page p of the unit (0..3).  b ==
// rows marks the end.  len is the row's current context length.
struct Task {
  int32_t b, u, p, len;
};

// Task iterator: the single definition of "what comes next" used by both the
// K lookahead and the consumer.
struct Iter {
  SchedView v;
  const int32_t* ctx;
  int32_t end_b, end_u;
  int32_t max_ctx;

  __device__ __forceinline__ bool in_range(int32_t b, int32_t u) const {
    return b < v.rows && (b < end_b || (b == end_b && u < end_u));
  }
  __device__ __forceinline__ Task make(int32_t b, int32_t u) const {
    Task t;
    if (in_range(b, u)) {
      t.b = b;
      t.u = u;
      t.p = 0;
      t.len = sload(ctx + b);
    } else {
      t.b = v.rows;
      t.u = t.p = t.len = 0;
    }
    return t;
  }
  // Next unit after (b, u), skipping rows that have no unit.
  __device__ __forceinline__ Task next_unit(int32_t b, int32_t u) const {
    if (u + 1 < units_of(v, b)) return make(b, u + 1);
    ++b;
    while (b < v.rows && units_of(v, b) == 0) ++b;
    return make(b, 0);
  }
  __device__ __forceinline__ Task first(int32_t b, int32_t u) const {
    b = min(max(b, 0), v.rows);
    u = max(u, 0);
    while (b < v.rows && u >= units_of(v, b)) {
      ++b;
      u = 0;
    }
    return make(b, u);
  }
  __device__ __forceinline__ Task next(const Task& t) const {
    const int32_t np = t.p + 1;
    if (np < kPagesPerUnit && t.u * kUnit + np * kPage < max_ctx) {
      Task n = t;
      n.p = np;
      return n;
    }
    return next_unit(t.b, t.u);
  }
  __device__ __forceinline__ bool valid(const Task& t) const { return t.b < v.rows; }
};

__device__ __forceinline__ int32_t page_token0(const Task& t) { return t.u * kUnit + t.p * kPage; }

// Does the page hold K data that some query row scores?
__device__ __forceinline__ bool has_data(const Task& t, const LogitsArgs& a) {
  return page_token0(t) < min(t.len, a.max_ctx) &&
         (t.u * kPagesPerUnit + t.p) < a.bt_stride;
}

__device__ __forceinline__ const uint8_t* page_ptr(const Task& t, const LogitsArgs& a,
                                                   int page_bytes) {
  const int32_t idx = t.u * kPagesPerUnit + t.p;
  int64_t pid = sload(a.bt + (int64_t)t.b * a.bt_stride + idx);
  pid = pid < 0 ? 0 : (pid >= a.num_pages ? a.num_pages - 1 : pid);
  return a.kv + pid * (int64_t)page_bytes;
}

// Reduce four per-lane partial sums (token group tg = 0..3 of lane-group
// partial head sums) across the four 16-lane groups; lane l returns the full
// sum for token l of the page.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
  auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false,
                                              false);
  auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false,
                                              false);
  const float a0 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
  const float a1 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
  auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a0), __float_as_uint(a1), false,
                                              false);
  return __uint_as_float(s01[0]) + __uint_as_float(s01[1]);
}

// Tail fill: -inf over the 256-column chunks at or past each row's unit
// count, split evenly over all workers.
__device__ __forceinline__ void fill_tail(const LogitsArgs& a, const SchedView& v, int next_n,
                                          int32_t wid, int lane) {
  const int32_t cm = v.cap;
  const int64_t rows = (int64_t)a.batch * next_n;
  const int64_t total = rows * cm;
  int64_t idx = ((int64_t)wid * total) / a.num_workers;
  const int64_t hi = ((int64_t)(wid + 1) * total) / a.num_workers;
  if (idx >= hi) return;
  int64_t r = idx / cm;
  int32_t k = (int32_t)(idx - r * cm);
  const float ninf = -__builtin_inff();
  const v4f nv = {ninf, ninf, ninf, ninf};
  while (idx < hi) {
    const int32_t b = (int32_t)(r / next_n);
    const int32_t c = b < v.rows ? units_of(v, b) : 0;
    if (k < c) {  // chunk written by the unit pass: jump past the row's units
      const int64_t skip = min((int64_t)(c - k), hi - idx);
      idx += skip;
      k += (int32_t)skip;
    } else {
      const int32_t col = k * kUnit + 4 * lane;
      float* dst = a.out + r * a.ldo + col;
      if (col + 4 <= a.max_ctx) {
        __builtin_nontemporal_store(nv, reinterpret_cast<v4f*>(dst));
      } else {
        for (int e = 0; e < 4; ++e)
          if (col + e < a.max_ctx) dst[e] = ninf;
      }
      ++idx;
      ++k;
    }
    if (k >= cm) {
      ++r;
      k = 0;
    }
  }
}

}  // namespace pmqa

namespace pmqa {

// Element-format policies -------------------------------------------------

// fp8: E4M3 q and K, per-token fp32 K scale applied in the epilogue.
struct Fp8Format {
  static constexpr int kPageBytes = kFp8PageBytes;
  static constexpr bool kTokenScale = true;
  struct KFrag {
    v8i k[4];
    float s;  // scale of token `lane` of the page
  };
  template <int NN>
  struct QFrag {
    v8i q[NN][4];
  };
  __device__ __forceinline__ static void load_k(const uint8_t* pg, int lane, KFrag& f) {
    const int c = lane >> 4, tl = lane & 15;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const v4i* src = reinterpret_cast<const v4i*>(pg + (16 * tg + tl) * kHeadDim + 32 * c);
      const v4i lo = src[0];
      const v4i hi = src[1];
      f.k[tg] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    f.s = reinterpret_cast<const float*>(pg + kPage * kHeadDim)[lane];
  }
  template <int NN>
  __device__ __forceinline__ static void load_q(const LogitsArgs& a, int32_t b, int lane,
                                                QFrag<NN>& q) {
    const int c = lane >> 4, tl = lane & 15;
#pragma unroll
    for (int j = 0; j < NN; ++j)
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) {
        const int64_t row = ((int64_t)b * NN + j) * kHeads + 16 * hg + tl;
        const v4i* src = reinterpret_cast<const v4i*>(a.q + row * kHeadDim + 32 * c);
        const v4i lo = src[0];
        const v4i hi = src[1];
        q.q[j][hg] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
  }
  template <int NN>
  __device__ __forceinline__ static v4f mma(const QFrag<NN>& q, int j, int hg, const KFrag& f,
                                            int tg) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.q[j][hg], f.k[tg], zero, kFmtFp8,
                                                            kFmtFp8, 0, kScaleOne, 0, kScaleOne);
  }
};

// MXFP4: E2M1 q and K with one E8M0 scale per 32 elements, fed to the MFMA
// as per-lane block scales; no per-token scale.
struct Fp4Format {
  static constexpr int kPageBytes = kFp4PageBytes;
  static constexpr bool kTokenScale = false;
  struct KFrag {
    v4i k[4];
    int32_t sc[4];
  };
  template <int NN>
  struct QFrag {
    v4i q[NN][4];
    int32_t sc[NN][4];
  };
  __device__ __forceinline__ static void load_k(const uint8_t* pg, int lane, KFrag& f) {
    const int c = lane >> 4, tl = lane & 15;
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const int tok = 16 * tg + tl;
      f.k[tg] = *reinterpret_cast<const v4i*>(pg + tok * (kHeadDim / 2) + 16 * c);
      f.sc[tg] = pg[kPage * kHeadDim / 2 + tok * (kHeadDim / 32) + c];
    }
  }
  template <int NN>
  __device__ __forceinline__ static void load_q(const LogitsArgs& a, int32_t b, int lane,
                                                QFrag<NN>& q) {
    const int c = lane >> 4, tl = lane & 15;
#pragma unroll
    for (int j = 0; j < NN; ++j)
#pragma unroll
      for (int hg = 0; hg < 4; ++hg) {
        const int64_t row = ((int64_t)b * NN + j) * kHeads + 16 * hg + tl;
        q.q[j][hg] = *reinterpret_cast<const v4i*>(a.q + row * (kHeadDim / 2) + 16 * c);
        q.sc[j][hg] = a.q_scale[row * (kHeadDim / 32) + c];
      }
  }
  template <int NN>
  __device__ __forceinline__ static v4f mma(const QFrag<NN>& q, int j, int hg, const KFrag& f,
                                            int tg) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const v4i x = q.q[j][hg];
    const v4i y = f.k[tg];
    const v8i a8 = {x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    const v8i b8 = {y[0], y[1], y[2], y[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, zero, kFmtFp4, kFmtFp4, 0,
                                                            q.sc[j][hg], 0, f.sc[tg]);
  }
};

// Per-row operands held in registers while a worker stays on one batch row.
template <class Fmt, int NN>
struct RowState {
  typename Fmt::template QFrag<NN> q;
  v4f w[NN][4];  // weights of heads 16*hg + 4*(lane>>4) + i
  int32_t b;
};

template <class Fmt, int NN>
__device__ __forceinline__ void load_row(const LogitsArgs& a, int32_t b, int lane,
                                         RowState<Fmt, NN>& rs) {
  Fmt::template load_q<NN>(a, b, lane, rs.q);
  const int c = lane >> 4;
#pragma unroll
  for (int j = 0; j < NN; ++j)
#pragma unroll
    for (int hg = 0; hg < 4; ++hg)
      rs.w[j][hg] = *reinterpret_cast<const v4f*>(a.weights + ((int64_t)b * NN + j) * kHeads +
                                                  16 * hg + 4 * c);
  rs.b = b;
}

// Contract one page against every query row of the batch row, apply the
// epilogue and store the page's 64 columns of each output row.
template <class Fmt, int NN>
__device__ __forceinline__ void process_page(const Task& t, const typename Fmt::KFrag& f,
                                             RowState<Fmt, NN>& rs, const LogitsArgs& a,
                                             int lane) {
  if (t.b != rs.b) load_row<Fmt, NN>(a, t.b, lane, rs);
  const int32_t tok = page_token0(t) + lane;
  const float ninf = -__builtin_inff();
  float val[NN];
#pragma unroll
  for (int j = 0; j < NN; ++j) val[j] = ninf;
  if (has_data(t, a)) {
    const int tl = lane & 15;
    uint64_t neg = 0;
    if constexpr (Fmt::kTokenScale) neg = __ballot(f.s < 0.f);
    float part[NN][4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const float bnd = ((neg >> (16 * tg + tl)) & 1) ? ninf : __builtin_inff();
#pragma unroll
      for (int j = 0; j < NN; ++j) {
        float sum = 0.f;
#pragma unroll
        for (int hg = 0; hg < 4; ++hg) {
          const v4f acc = Fmt::template mma<NN>(rs.q, j, hg, f, tg);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sum = __builtin_fmaf(rs.w[j][hg][i], __builtin_amdgcn_fmed3f(acc[i], 0.f, bnd), sum);
        }
        part[j][tg] = sum;
      }
    }
#pragma unroll
    for (int j = 0; j < NN; ++j) {
      float tot = reduce_scatter4(part[j][0], part[j][1], part[j][2], part[j][3]);
      if constexpr (Fmt::kTokenScale) tot *= f.s;
      val[j] = tot;
    }
  }
  if (tok < a.max_ctx) {
#pragma unroll
    for (int j = 0; j < NN; ++j) {
      const int32_t lim = t.len - NN + 1 + j;
      const int64_t r = (int64_t)t.b * NN + j;
      a.out[r * a.ldo + tok] = tok < lim ? val[j] : ninf;
    }
  }
}

__device__ __forceinline__ int32_t xcd_block(int32_t bid, int32_t nblk) {
  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
  // contiguous range of workers so neighbouring units share its L2.
  constexpr int32_t kXcds = 8;
  if (nblk % kXcds) return bid;
  return (bid % kXcds) * (nblk / kXcds) + bid / kXcds;
}

template <class Fmt, int NN>
__global__ __launch_bounds__(kBlockThreads) void logits_kernel(const LogitsArgs a) {
  const int lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wid = xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wave;
  if (wid >= a.num_workers) return;
  const SchedView v = make_view(a);
  if (v.rows > 0) {
    Iter it;
    it.v = v;
    it.ctx = a.ctx;
    it.end_b = sload(v.starts + 2 * wid + 2);
    it.end_u = sload(v.starts + 2 * wid + 3);
    it.max_ctx = a.max_ctx;
    Task cur = it.first(sload(v.starts + 2 * wid), sload(v.starts + 2 * wid + 1));
    typename Fmt::KFrag fa, fb;
    RowState<Fmt, NN> rs;
    rs.b = -1;
    if (it.valid(cur) && has_data(cur, a))
      Fmt::load_k(page_ptr(cur, a, Fmt::kPageBytes), lane, fa);
    while (it.valid(cur)) {
      const Task nx = it.next(cur);
      if (it.valid(nx) && has_data(nx, a))
        Fmt::load_k(page_ptr(nx, a, Fmt::kPageBytes), lane, fb);
      process_page<Fmt, NN>(cur, fa, rs, a, lane);
      if (!it.valid(nx)) break;
      cur = it.next(nx);
      if (it.valid(cur) && has_data(cur, a))
        Fmt::load_k(page_ptr(cur, a, Fmt::kPageBytes), lane, fa);
      process_page<Fmt, NN>(nx, fb, rs, a, lane);
    }
  }
  fill_tail(a, v, NN, wid, lane);
}

template <class Fmt>
hipError_t launch_logits(const LogitsArgs& a, int next_n, hipStream_t stream) {
  const dim3 grid((a.num_workers + kWavesPerBlock - 1) / kWavesPerBlock);
  const dim3 block(kBlockThreads);
  if (next_n == 1)
    hipLaunchKernelGGL((logits_kernel<Fmt, 1>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((logits_kernel<Fmt, 2>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <class Fmt>
hipError_t blocks_per_cu(int next_n, int* blocks) {
  if (next_n == 1)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, logits_kernel<Fmt, 1>,
                                                        kBlockThreads, 0);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, logits_kernel<Fmt, 2>,
                                                      kBlockThreads, 0);
}

}  // namespace pmqa
