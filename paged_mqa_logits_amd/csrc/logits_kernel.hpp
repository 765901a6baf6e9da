// Persistent paged MQA logits kernel for gfx950, shared by the fp8 and MXFP4
// element formats.
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입":
// introduction (the indexer score: ReLU of each head's score, weighted
// per head and summed; fp8 and fp4 kernels), section 1 (the task iterator skips zero-length rows) and the
// general lessons (lookahead and the task iterator must pick the same rows).
//
// Mapping onto CDNA4
// ------------------
// One worker is one 64-lane wavefront.  A worker walks its schedule range of
// 256-token units; a unit is 4 pages of 64 tokens.  For a page it contracts
// the 64-head query block of each query row against the page's 64 K rows with
// v_mfma_scale_f32_16x16x128_f8f6f4: K = head_dim = 128 is covered by one
// instruction, so a page is 4 head groups x 4 token groups x next_n MFMAs.
//
//   A operand (query): lane l holds head 16*hg + (l & 15), elements
//     [32*(l>>4), +32) of head_dim.  Loaded once per batch row.
//   B operand (K):     lane l holds token 16*tg + (l & 15), the same element
//     range.  Every K byte is used by exactly one lane.  A page is read with
//     contiguous 16-byte non-temporal loads (1 KB per instruction, which
//     streams faster than loading in operand order) and reordered into the
//     operand layout through a small LDS buffer of the wavefront's own (the
//     element-format policies below).
//   C (scores):        lane l holds heads 16*hg + 4*(l>>4) + i, i = 0..3, of
//     token 16*tg + (l & 15).
//
// Epilogue per (head, token): one v_med3 (ReLU, or its mirror for a negative
// token scale) and one FMA with the head weight; the 16 heads of a lane are
// summed in registers, then the four lane groups are reduced and scattered
// with permlane32/permlane16 swaps so that lane l ends up owning token l of
// the page and the 64 results are stored as one contiguous 256-byte row.
//
// Memory pipeline
// ---------------
// One worker wavefront runs per SIMD for fp8 (two for MXFP4, whose pages
// are half the bytes), which leaves registers for a ring of 4 K pages: while
// a unit's 4 pages are consumed, the next unit's 4 pages are in flight.
// K pages are read through buffer resources.  A page with no data to score
// (past the context, or past the block table) gets a zero-size resource, so
// its loads return zeros without touching memory, and output rows are stored
// through a resource sized to max_context_len, so columns past it are dropped
// by the hardware.  Every page therefore issues the same memory instructions,
// which lets the compiler wait for exactly the page being consumed while the
// next one is in flight (double buffering in VGPRs).  The block-table entries
// of the next unit are requested at the start of the current one.  The
// lookahead and the consumer walk the same iterator, so they always agree on
// which (row, unit) comes next, including across skipped zero-length rows.
//
// Finished logits are staged in LDS and written in bursts, at moments
// shared by all workers (see Stage below).  Every output column is first set
// to -inf by a separate kernel (tail_fill.hip) launched right before this
// one; this kernel overwrites the columns of the units it processes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pmqa_internal.h"

namespace pmqa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kFmtFp8 = 0;      // cbsz/blgp code of E4M3 operands
constexpr int kFmtFp4 = 4;      // cbsz/blgp code of E2M1 operands
constexpr int kScaleOne = 127;  // E8M0 encoding of 1.0
// Word 3 of a raw buffer resource on gfx9-class GPUs (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy bits of a streaming (non-temporal) buffer load.
constexpr int kLoadNT = 2;
// Cache-policy bits of a non-temporal store.
constexpr int kStoreNT = 2;
// Cache-policy bits of the logit stores: SC1 (device scope).  Measured on
// MI355X, stores issued this way slow the K stream less than plain or
// non-temporal ones (large_fp8 call -6 us, mxfp4 -14 us).
constexpr int kStoreSc1 = 16;

// Wave-uniform read of read-only metadata (schedule, context lengths, block
// table) through the constant address space, so it is a scalar load that
// waits on lgkmcnt only and never on the vector loads in flight.
typedef const __attribute__((address_space(4))) int32_t* cint_ptr;

__device__ __forceinline__ int32_t sload(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane(*(cint_ptr)(p));
}

// bytes is the unsigned 32-bit record count (up to 2^32 - 1).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int32_t)bytes,
                                           kRsrcWord3);
}

// Read-only view of a schedule; every index derived from it is clamped.
struct SchedView {
  const int32_t* starts;
  const int32_t* S;
  int32_t rows;  // batch rows covered (0 when the schedule is unusable)
  int32_t cap;   // units per row never exceed ceil(max_ctx / 256)
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

// One unit of work: batch row b, unit u (tokens [256u, 256u + 256)).
// b == rows marks the end.  len is the row's current context length, units
// its unit count, raw the block-table entries of the unit's 4 pages as read
// (validated and clamped only where they are used, so the scalar loads that
// fetch them one unit ahead are not waited for early).
struct Unit {
  int32_t b, u, len, units;
  int32_t raw[kPagesPerUnit];
};

// Task iterator: the single definition of "what comes next", used both for
// the lookahead (block-table entries and first page of the next unit) and
// for the unit being consumed.
struct Iter {
  SchedView v;
  const LogitsArgs* a;
  int32_t end_b, end_u;

  __device__ __forceinline__ bool valid(const Unit& t) const { return t.b < v.rows; }

  __device__ __forceinline__ Unit make(int32_t b, int32_t u, int32_t len, int32_t units) const {
    Unit t;
    const bool in = b < v.rows && (b < end_b || (b == end_b && u < end_u));
    t.b = in ? b : v.rows;
    t.u = u;
    t.len = len;
    t.units = units;
    // Unconditional loads of in-bounds entries: the row index is clamped to
    // the table and the column to the row, whatever the unit holds.
    const int32_t bb = min(b, a->batch - 1);
    const int64_t row = (int64_t)bb * a->bt_stride;
#pragma unroll
    for (int p = 0; p < kPagesPerUnit; ++p)
      t.raw[p] = sload(a->bt + row + min(u * kPagesPerUnit + p, a->bt_stride - 1));
    return t;
  }
  __device__ __forceinline__ Unit enter_row(int32_t b, int32_t u) const {
    if (b >= v.rows) return make(v.rows, 0, 0, 0);
    return make(b, u, sload(a->ctx + b), units_of(v, b));
  }
  // First unit of the worker, from its schedule start (clamped).  A start
  // names a unit of its row, so the row's prefix sums, length and
  // block-table entries are all requested at once (one round trip of
  // scalar loads); the loop is for starts that do not.
  __device__ __forceinline__ Unit first(int32_t b, int32_t u) const {
    b = min(max(b, 0), v.rows);
    u = max(u, 0);
    const int32_t bb = min(b, a->batch - 1);
    Unit t = make(b, u, 0, 0);  // block-table entries first: nothing they need is loaded
    const int32_t s0 = sload(v.S + bb), s1 = sload(v.S + bb + 1), len = sload(a->ctx + bb);
    __asm__ volatile("" ::"s"(s0), "s"(s1), "s"(len), "s"(t.raw[0]), "s"(t.raw[1]),
                     "s"(t.raw[2]), "s"(t.raw[3]));
    t.len = len;
    t.units = min(max(s1 - s0, 0), v.cap);
    if (b >= v.rows || u < t.units) return t;
    while (b < v.rows && u >= units_of(v, b)) {
      ++b;
      u = 0;
    }
    return enter_row(b, u);
  }
  // Next unit after t, skipping rows that have no unit.
  __device__ __forceinline__ Unit next(const Unit& t) const {
    if (t.u + 1 < t.units) return make(t.b, t.u + 1, t.len, t.units);
    int32_t b = t.b + 1;
    while (b < v.rows && units_of(v, b) == 0) ++b;
    return enter_row(b, 0);
  }
};

// Does page p of unit t hold K data that some query row scores?  (Token
// start below min(len, max_ctx), entry inside the block table.)
__device__ __forceinline__ bool page_has_data(const Unit& t, int p, const LogitsArgs& a,
                                              int32_t rows) {
  const int32_t idx = t.u * kPagesPerUnit + p;
  return t.b < rows && idx * kPage < min(t.len, a.max_ctx) && idx < a.bt_stride;
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

// Element-format policies -------------------------------------------------

// fp8: E4M3 q and K, per-token fp32 K scale applied in the epilogue.
//
// A page's 8 KB of K values are read with contiguous, non-temporal 16-byte
// loads (each load instruction covers 1 KB: eight full 128-byte lines of 8
// tokens), which streams faster from HBM than loading straight in MFMA
// operand order (16 half-lines per instruction).  Before the page is
// contracted it is passed through the wave's 8 KB LDS buffer to reach the
// operand layout.  In LDS, 16-byte chunk k of token t sits at
// t*128 + ((k ^ ((t >> 1) & 7)) << 4): the 1 KB written by each store
// instruction stays contiguous, and the 16 lanes of each operand read hit 16
// distinct bank groups.
struct Fp8Format {
  static constexpr int kPageBytes = kFp8PageBytes;
  static constexpr bool kTokenScale = true;
  static constexpr int kLdsBytes = kPage * kHeadDim;  // transpose buffer per wave
  // Waves per SIMD (one: the stream is memory-bound and the registers go to
  // the K ring) and units of logits staged per wave.  With 32 or 16 heads
  // the smaller query block and accumulators would let two waves fit, but
  // that halves the stage (two workgroups in LDS), and measured on MI355X
  // the longer write bursts of one wave per SIMD win.
  static constexpr int waves_per_simd(int, int) { return 1; }
  static constexpr int stage_units(int nn, int) { return 28 / nn; }
  struct KFrag {
    v4i raw[8];  // raw[i]: bytes [1024 i + 16 lane, +16) of the page's values
    float s;     // scale of token `lane` of the page
  };
  struct KOp {
    v8i k[4];    // MFMA B operand of token group tg
  };
  template <int NN, int HG>
  struct QFrag {
    v8i q[NN][HG];
  };
  __device__ __forceinline__ static void load_k(rsrc_t pg, int lane, KFrag& f) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      f.raw[i] = __builtin_amdgcn_raw_buffer_load_b128(pg, 1024 * i + 16 * lane, 0, kLoadNT);
    f.s = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(pg, kPage * kHeadDim + 4 * lane, 0, 0));
  }
  // Reorder a page into operand layout through the wave's LDS buffer.
  __device__ __forceinline__ static void to_operands(const KFrag& f, uint8_t* lds, int lane,
                                                     KOp& o) {
    // store i writes tokens 8i + (lane >> 3), chunk lane & 7; the swizzle of
    // token t = 8i + (lane >> 3) is (4i + (lane >> 4)) & 7
    const int tok_in = lane >> 3;
    const int w_even = tok_in * 128 + (((lane & 7) ^ ((lane >> 4) & 7)) << 4);
    const int w_odd = tok_in * 128 + (((lane & 7) ^ ((4 + (lane >> 4)) & 7)) << 4);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<v4i*>(lds + 1024 * i + ((i & 1) ? w_odd : w_even)) = f.raw[i];
    // operand lane (tl, c) of group tg wants token 16 tg + tl, chunks 2c, 2c+1
    const int tl = lane & 15, c = lane >> 4;
    const int sw = (tl >> 1) & 7;
    const int r0 = tl * 128 + (((2 * c) ^ sw) << 4);
    const int r1 = tl * 128 + (((2 * c + 1) ^ sw) << 4);
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const v4i lo = *reinterpret_cast<const v4i*>(lds + 2048 * tg + r0);
      const v4i hi = *reinterpret_cast<const v4i*>(lds + 2048 * tg + r1);
      o.k[tg] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  template <int NN, int HG>
  __device__ __forceinline__ static void load_q(const LogitsArgs& a, int32_t b, int lane,
                                                QFrag<NN, HG>& q) {
    const int c = lane >> 4, tl = lane & 15;
#pragma unroll
    for (int j = 0; j < NN; ++j)
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const int64_t row = ((int64_t)b * NN + j) * (16 * HG) + 16 * hg + tl;
        const v4i* src = reinterpret_cast<const v4i*>(a.q + row * kHeadDim + 32 * c);
        const v4i lo = src[0];
        const v4i hi = src[1];
        q.q[j][hg] = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
  }
  template <int NN, int HG>
  __device__ __forceinline__ static v4f mma(const QFrag<NN, HG>& q, int j, int hg,
                                            const KOp& o, int tg) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.q[j][hg], o.k[tg], zero, kFmtFp8,
                                                            kFmtFp8, 0, kScaleOne, 0, kScaleOne);
  }
};

// MXFP4: E2M1 q and K with one E8M0 scale per 32 elements, fed to the MFMA
// as per-lane block scales; no per-token scale.
//
// As for fp8, a page's 4 KB of packed values are read with contiguous
// non-temporal 16-byte loads (1 KB, i.e. 16 tokens, per instruction) and
// reordered to operand layout through the wave's LDS buffer: chunk k (16
// bytes = 32 elements) of token t sits at t*64 + ((k ^ ((t >> 2) & 3)) << 4),
// which keeps stores and operand reads free of bank conflicts.  Lane l also
// loads the four block scales of token l, and each operand lane fetches the
// scale it needs from the owning lane with ds_bpermute.
struct Fp4Format {
  static constexpr int kPageBytes = kFp4PageBytes;
  static constexpr bool kTokenScale = false;
  static constexpr int kLdsBytes = kPage * kHeadDim / 2;  // transpose buffer per wave
  // Two waves per SIMD (a page costs as many MFMA and VALU issues as an fp8
  // page for half the bytes, so a second wave fills the issue gaps of the
  // first), with the logits stage halved to fit two workgroups in LDS.
  static constexpr int waves_per_simd(int, int) { return 2; }
  static constexpr int stage_units(int nn, int) { return 14 / nn; }
  struct KFrag {
    v4i raw[4];   // raw[i]: bytes [1024 i + 16 lane, +16) of the page's values
    int32_t sc;   // the 4 E8M0 block scales of token `lane`
  };
  struct KOp {
    v4i k[4];     // B operand of token group tg (16 bytes = 32 elements)
    int32_t sc[4];
  };
  template <int NN, int HG>
  struct QFrag {
    v4i q[NN][HG];
    int32_t sc[NN][HG];
  };
  __device__ __forceinline__ static void load_k(rsrc_t pg, int lane, KFrag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.raw[i] = __builtin_amdgcn_raw_buffer_load_b128(pg, 1024 * i + 16 * lane, 0, kLoadNT);
    f.sc = __builtin_amdgcn_raw_buffer_load_b32(pg, kPage * kHeadDim / 2 + 4 * lane, 0, 0);
  }
  __device__ __forceinline__ static void to_operands(const KFrag& f, uint8_t* lds, int lane,
                                                     KOp& o) {
    // store i writes token 16 i + (lane >> 2), chunk lane & 3; its swizzle is
    // (lane >> 4) & 3
    const int w = (lane >> 2) * 64 + (((lane & 3) ^ ((lane >> 4) & 3)) << 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(lds + 1024 * i + w) = f.raw[i];
    // operand lane (tl, c) of group tg wants token 16 tg + tl, chunk c
    const int tl = lane & 15, c = lane >> 4;
    const int r = tl * 64 + ((c ^ ((tl >> 2) & 3)) << 4);
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      o.k[tg] = *reinterpret_cast<const v4i*>(lds + 1024 * tg + r);
      const int owner = __builtin_amdgcn_ds_bpermute(4 * (16 * tg + tl), f.sc);
      o.sc[tg] = (owner >> (8 * c)) & 0xFF;
    }
  }
  template <int NN, int HG>
  __device__ __forceinline__ static void load_q(const LogitsArgs& a, int32_t b, int lane,
                                                QFrag<NN, HG>& q) {
    const int c = lane >> 4, tl = lane & 15;
#pragma unroll
    for (int j = 0; j < NN; ++j)
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const int64_t row = ((int64_t)b * NN + j) * (16 * HG) + 16 * hg + tl;
        q.q[j][hg] = *reinterpret_cast<const v4i*>(a.q + row * (kHeadDim / 2) + 16 * c);
        q.sc[j][hg] = a.q_scale[row * (kHeadDim / 32) + c];
      }
  }
  template <int NN, int HG>
  __device__ __forceinline__ static v4f mma(const QFrag<NN, HG>& q, int j, int hg,
                                            const KOp& o, int tg) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const v4i x = q.q[j][hg];
    const v4i y = o.k[tg];
    const v8i a8 = {x[0], x[1], x[2], x[3], 0, 0, 0, 0};
    const v8i b8 = {y[0], y[1], y[2], y[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, zero, kFmtFp4, kFmtFp4, 0,
                                                            q.sc[j][hg], 0, o.sc[tg]);
  }
};

// Per-row operands held in registers while a worker stays on one batch row
// (HG groups of 16 heads).
template <class Fmt, int NN, int HG>
struct RowState {
  typename Fmt::template QFrag<NN, HG> q;
  v4f w[NN][HG];  // weights of heads 16*hg + 4*(lane>>4) + i
  int32_t b;
};

template <class Fmt, int NN, int HG>
__device__ __forceinline__ void load_row(const LogitsArgs& a, int32_t b, int lane,
                                         RowState<Fmt, NN, HG>& rs) {
  Fmt::template load_q<NN, HG>(a, b, lane, rs.q);
  const int c = lane >> 4;
#pragma unroll
  for (int j = 0; j < NN; ++j)
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
      rs.w[j][hg] = *reinterpret_cast<const v4f*>(
          a.weights + ((int64_t)b * NN + j) * (16 * HG) + 16 * hg + 4 * c);
  rs.b = b;
}

template <class Fmt>
__device__ __forceinline__ void load_page(const LogitsArgs& a, const Unit& t, int p, int32_t rows,
                                          int lane, typename Fmt::KFrag& f) {
  const bool ok = page_has_data(t, p, a, rows);
  int64_t pid = t.raw[p];
  pid = pid < 0 ? 0 : (pid >= a.num_pages ? a.num_pages - 1 : pid);
  const uint8_t* base = a.kv + (ok ? pid : 0) * Fmt::kPageBytes;
  Fmt::load_k(make_rsrc(base, ok ? Fmt::kPageBytes : 0), lane, f);
}

// Contract page p of unit t against every query row of the batch row and
// apply the epilogue; lane l returns the logit of token l of the page for
// each query row (-inf past the row's causal limit).
template <class Fmt, int NN, int HG>
__device__ __forceinline__ void process_page(const Unit& t, int p, const typename Fmt::KFrag& f,
                                             uint8_t* lds, const RowState<Fmt, NN, HG>& rs,
                                             const LogitsArgs& a, int32_t rows, int lane,
                                             float (&res)[NN]) {
  const int32_t tok = t.u * kUnit + p * kPage + lane;
  const float ninf = -__builtin_inff();
  float val[NN];
#pragma unroll
  for (int j = 0; j < NN; ++j) val[j] = ninf;
  if (page_has_data(t, p, a, rows)) {
    const int tl = lane & 15;
    typename Fmt::KOp op;
    Fmt::to_operands(f, lds, lane, op);
    uint64_t neg = 0;
    if constexpr (Fmt::kTokenScale) neg = __ballot(f.s < 0.f);
    // Upper clamp of the ReLU: +inf, or -inf for a token whose scale is
    // negative (ReLU(s*x) = s*min(x, 0) then, the scale being applied after
    // the head sum).  Kept opaque when it is a constant so the ReLU stays one
    // med3 instead of a max that the compiler precedes with a NaN-quieting
    // max(x, x).
    float pos = __builtin_inff();
    if constexpr (!Fmt::kTokenScale) __asm__("" : "+v"(pos));
    float part[NN][4];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const float bnd = ((neg >> (16 * tg + tl)) & 1) ? ninf : pos;
      v4f acc[NN][HG];
#pragma unroll
      for (int j = 0; j < NN; ++j)
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
          acc[j][hg] = Fmt::template mma<NN, HG>(rs.q, j, hg, op, tg);
#pragma unroll
      for (int j = 0; j < NN; ++j) {
        float sum = 0.f;
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sum = __builtin_fmaf(rs.w[j][hg][i], __builtin_amdgcn_fmed3f(acc[j][hg][i], 0.f, bnd),
                                 sum);
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
#pragma unroll
  for (int j = 0; j < NN; ++j) res[j] = tok < t.len - NN + 1 + j ? val[j] : ninf;
}

__device__ __forceinline__ int32_t xcd_block(int32_t bid, int32_t nblk) {
  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
  // contiguous range of workers so neighbouring units share its L2.
  constexpr int32_t kXcds = 8;
  if (nblk % kXcds) return bid;
  return (bid % kXcds) * (nblk / kXcds) + bid / kXcds;
}

// Staging of finished logits: every worker keeps the results of its last
// kUnits units in LDS (256 floats per unit and query row) and writes them
// out together, 16 bytes per lane.  Writing in a few large bursts instead of
// 256 bytes after every page keeps most of the output traffic out of the
// read stream.  The stage takes what LDS is left once the format's
// workgroups per compute unit are resident.
//
// When to flush: at the end, when the stage is full, and at the first unit
// boundary after each tick of a chip-wide clock (s_memrealtime, 100 MHz,
// the same counter on every compute unit) crosses a multiple of
// flush_ticks, provided a quarter of the stage is filled.  All workers
// then write at about the same time, so HBM sees dense write bursts between
// long read-only stretches instead of a trickle of writes mixed into the K
// stream.  The period is sized so that a worker streaming its share of
// ~6 TB/s fills about 65% of its stage per period (a worker running slower
// flushes fewer units; one running faster fills the stage and flushes on
// its own).  Measured on MI355X against flushing only full stages: mxfp4
// call -26 us, large_fp8 -4 us.
template <class Fmt, int NN, int HG>
struct Stage {
  static constexpr int kUnits = Fmt::stage_units(NN, HG);
  static constexpr int kFloats = kUnits * NN * kUnit;
  static constexpr int kMinPhaseUnits = (kUnits + 3) / 4;
};

constexpr double kStreamBytesPerTick = 6.0e12 / 1.0e8;  // K bytes per 100 MHz tick, all workers
constexpr double kPhaseFill = 0.65;                    // stage fraction filled per period

template <class Fmt, int NN, int HG>
uint32_t flush_period_ticks(int32_t workers) {
  const double unit_ticks =
      (double)Fmt::kPageBytes * kPagesPerUnit * (double)(workers > 0 ? workers : 1) /
      kStreamBytesPerTick;
  const double t = kPhaseFill * Stage<Fmt, NN, HG>::kUnits * unit_ticks;
  return t < 1.0 ? 1u : t > 4.0e9 ? 4000000000u : (uint32_t)t;
}

// Index of the current flush period (the low 32 bits of the clock wrap every
// 43 s; a wrap only adds one early flush).
__device__ __forceinline__ uint32_t flush_phase(uint32_t period) {
  return (uint32_t)__builtin_amdgcn_s_memrealtime() / period;
}

template <int NN>
__device__ __forceinline__ void flush_stage(const LogitsArgs& a, const float* stage,
                                            const int32_t* meta, int32_t n, int lane) {
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = __builtin_amdgcn_readfirstlane(meta[2 * i]);
    const int32_t u = __builtin_amdgcn_readfirstlane(meta[2 * i + 1]);
    const int32_t col = u * kUnit + 4 * lane;
#pragma unroll
    for (int j = 0; j < NN; ++j) {
      const int64_t r = (int64_t)b * NN + j;
      const v4f v = *reinterpret_cast<const v4f*>(stage + (i * NN + j) * kUnit + 4 * lane);
      const rsrc_t orow = make_rsrc(a.out + r * a.ldo, 4u * (uint32_t)a.max_ctx);
      if (u * kUnit + kUnit <= a.max_ctx) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), orow,
                                               (int32_t)(4u * (uint32_t)col), 0, kStoreSc1);
      } else {  // unit crosses max_ctx: per-column stores, the rest is dropped
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v[e]), orow,
                                                (int32_t)(4u * (uint32_t)(col + e)), 0, kStoreSc1);
      }
    }
  }
}

// -inf over piece `piece` of `pieces` of output row r's columns that no
// unit covers ([256 c_b, max_ctx), c_b the unit count of its batch row b
// from prefix sums s0 = S[b], s1 = S[b+1]; the whole row when the schedule
// is unusable).  Used for small outputs instead of the separate fill kernel:
// those columns are disjoint from every unit's, so no order is needed.
__device__ __forceinline__ void fill_tail(const LogitsArgs& a, const SchedView& v, int32_t r,
                                          int32_t piece, int32_t pieces, int32_t s0,
                                          int32_t s1, int lane) {
  const int32_t c = v.rows ? min(max(s1 - s0, 0), v.cap) : 0;
  const int32_t start = min(c * kUnit, a.max_ctx);
  const int32_t per = ((a.max_ctx - start + pieces - 1) / pieces + 3) & ~3;
  const int32_t c0 = min(a.max_ctx, start + piece * per), c1 = min(a.max_ctx, c0 + per);
  const rsrc_t orow = make_rsrc(a.out + (int64_t)r * a.ldo, 4u * (uint32_t)a.max_ctx);
  const float ninf = -__builtin_inff();
  const v4f nv = {ninf, ninf, ninf, ninf};
  for (int32_t col = c0 + 4 * lane; col < c1; col += 256) {
    if (col + 4 <= c1) {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, nv), orow,
                                             (int32_t)(4u * (uint32_t)col), 0, kStoreNT);
    } else {
      for (int e = 0; e < 4; ++e)
        if (col + e < c1)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(ninf), orow,
                                                (int32_t)(4u * (uint32_t)(col + e)), 0, kStoreNT);
    }
  }
}

template <class Fmt, int NN, int HG>
__global__ __launch_bounds__(kBlockThreads)
__attribute__((amdgpu_waves_per_eu(Fmt::waves_per_simd(NN, HG), Fmt::waves_per_simd(NN, HG))))
void logits_kernel(const LogitsArgs a) {
  __shared__ float stage_all[kWavesPerBlock][Stage<Fmt, NN, HG>::kFloats];
  __shared__ int32_t meta_all[kWavesPerBlock][2 * Stage<Fmt, NN, HG>::kUnits];
  __shared__ __attribute__((aligned(16))) uint8_t xpose_all[kWavesPerBlock][Fmt::kLdsBytes > 0 ? Fmt::kLdsBytes : 16];
  const int lane = threadIdx.x & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t wid = xcd_block(blockIdx.x, gridDim.x) * kWavesPerBlock + wave;
  if (wid >= a.num_workers) return;
  // The worker's range is requested together with the header (a buffer
  // for this call's batch and worker count holds it, whatever the header
  // says): one round trip.  The empty asm takes every value, so that no
  // load is sunk below the first use of another.
  const int32_t* range = a.sched + kSchedHeader + 2 * wid;
  const int32_t start_b = sload(range), start_u = sload(range + 1);
  const int32_t end_b = sload(range + 2), end_u = sload(range + 3);
  const SchedView v = make_view(a);
  // Small outputs: the workers also write -inf past every row's units, the
  // R output rows dealt out as R * (W / R) pieces (R <= W, checked by the
  // launcher); the prefix sums of the piece's row come with the range.
  const int32_t out_rows = a.batch * NN;
  const int32_t fr = wid % out_rows, fpiece = wid / out_rows;
  const int32_t fpieces = a.num_workers / out_rows;
  const bool fill = a.fill_tails && fpiece < fpieces;
  const int32_t fs0 = fill ? sload(v.S + fr / NN) : 0;
  const int32_t fs1 = fill ? sload(v.S + fr / NN + 1) : 0;
  __asm__ volatile("" ::"s"(start_b), "s"(start_u), "s"(end_b), "s"(end_u), "s"(v.rows),
                   "s"(fs0), "s"(fs1));
  if (v.rows == 0) {
    if (fill) fill_tail(a, v, fr, fpiece, fpieces, fs0, fs1, lane);
    return;
  }
  float* stage = stage_all[wave];
  int32_t* meta = meta_all[wave];
  uint8_t* xpose = xpose_all[wave];
  Iter it;
  it.v = v;
  it.a = &a;
  it.end_b = end_b;
  it.end_u = end_u;
  Unit cur = it.first(start_b, start_u);
  if (!it.valid(cur)) {
    if (fill) fill_tail(a, v, fr, fpiece, fpieces, fs0, fs1, lane);
    return;
  }
  const int32_t rows = v.rows;
  // The first row's query block and weights are requested before the first
  // pages, so waiting for them does not wait for the pages too.
  RowState<Fmt, NN, HG> rs;
  load_row<Fmt, NN, HG>(a, cur.b, lane, rs);
  // K ring: page p of a unit always lives in slot p, so the 4 pages of the
  // next unit are in flight while the current one is consumed.
  typename Fmt::KFrag ring[kPagesPerUnit];
#pragma unroll
  for (int p = 0; p < kPagesPerUnit; ++p) load_page<Fmt>(a, cur, p, rows, lane, ring[p]);
  // the -inf stores go out while the first pages are on their way
  if (fill) fill_tail(a, v, fr, fpiece, fpieces, fs0, fs1, lane);
  int32_t staged = 0;
  uint32_t phase = flush_phase(a.flush_ticks);
  // One exit, after the flush of the last unit, so the load counter has the
  // same history on every path into the loop head and each page waits only
  // for its own loads.
  while (true) {
    if (cur.b != rs.b) {  // new batch row: its query block and weights
      load_row<Fmt, NN, HG>(a, cur.b, lane, rs);
      __builtin_amdgcn_s_waitcnt(0);
    }
    const Unit nxt = it.next(cur);  // lookahead: same iterator as the consumer
    float* dst = stage + staged * NN * kUnit;
#pragma unroll
    for (int p = 0; p < kPagesPerUnit; ++p) {
      float res[NN];
      process_page<Fmt, NN, HG>(cur, p, ring[p], xpose, rs, a, rows, lane, res);
      load_page<Fmt>(a, nxt, p, rows, lane, ring[p]);
#pragma unroll
      for (int j = 0; j < NN; ++j) dst[j * kUnit + p * kPage + lane] = res[j];
    }
    if (lane == 0) {
      meta[2 * staged] = cur.b;
      meta[2 * staged + 1] = cur.u;
    }
    ++staged;
    const bool last = !it.valid(nxt);
    const uint32_t ph = flush_phase(a.flush_ticks);
    if (staged == Stage<Fmt, NN, HG>::kUnits || last ||
        (ph != phase && staged >= Stage<Fmt, NN, HG>::kMinPhaseUnits)) {
      phase = ph;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      flush_stage<NN>(a, stage, meta, staged, lane);
      __builtin_amdgcn_wave_barrier();
      staged = 0;
    }
    if (last) break;
    cur = nxt;
  }
}

template <class Fmt, int NN, int HG>
hipError_t launch_one(const LogitsArgs& a, hipStream_t stream) {
  const dim3 grid((a.num_workers + kWavesPerBlock - 1) / kWavesPerBlock);
  LogitsArgs b = a;
  b.flush_ticks = flush_period_ticks<Fmt, NN, HG>(a.num_workers);
  hipLaunchKernelGGL((logits_kernel<Fmt, NN, HG>), grid, dim3(kBlockThreads), 0, stream, b);
  return hipGetLastError();
}

// heads: 64, 32 or 16 (checked by the caller).
template <class Fmt>
hipError_t launch_logits(const LogitsArgs& a, int next_n, int heads, hipStream_t stream) {
  if (next_n == 1)
    return heads == 64 ? launch_one<Fmt, 1, 4>(a, stream)
                       : heads == 32 ? launch_one<Fmt, 1, 2>(a, stream)
                                     : launch_one<Fmt, 1, 1>(a, stream);
  return heads == 64 ? launch_one<Fmt, 2, 4>(a, stream)
                     : heads == 32 ? launch_one<Fmt, 2, 2>(a, stream)
                                   : launch_one<Fmt, 2, 1>(a, stream);
}

template <class Fmt, int NN, int HG>
hipError_t occupancy(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, logits_kernel<Fmt, NN, HG>,
                                                      kBlockThreads, 0);
}

template <class Fmt>
hipError_t blocks_per_cu(int next_n, int heads, int* blocks) {
  if (next_n == 1)
    return heads == 64 ? occupancy<Fmt, 1, 4>(blocks)
                       : heads == 32 ? occupancy<Fmt, 1, 2>(blocks) : occupancy<Fmt, 1, 1>(blocks);
  return heads == 64 ? occupancy<Fmt, 2, 4>(blocks)
                     : heads == 32 ? occupancy<Fmt, 2, 2>(blocks) : occupancy<Fmt, 2, 1>(blocks);
}

}  // namespace pmqa
