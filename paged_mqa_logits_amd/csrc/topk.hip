// Top-k token selection over rows of logits.
//
// Page "[flashinfer] Blackwell 아키텍처를 위한 고성능 Paged MQA Logits 커널 도입",
// introduction: the logits feed the indexer, which selects KV tokens by
// them.  The page gives neither k nor an order; the rule here is: a row's
// candidates are its first n columns, the selection is the k largest of
// them in the total order of fp32 values with -0 < +0 (no NaN), equal values
// ordered by column, lower first, and the selected columns are written in
// ascending order with their values; a row with n < k writes all n and pads
// with column -1, value -inf.
//
// Values are mapped to order-preserving 32-bit keys where ties and signed
// zeros matter; elsewhere they are compared and binned as floats.  Three
// ways to select a row, each exact:
//
//   * Rows of at most kWaveCols (6144) candidates, when there are more rows
//     than workgroups that fit on the chip at once (else only the rows
//     copied whole): one wavefront per row,
//     eight (512 threads) or sixteen (1024) rows to a workgroup, no
//     workgroup barrier.  The wavefront reads its row three times (the
//     first read from HBM, the others mostly from the caches): a histogram
//     of value-linear bins set from a 64-point sample of the row, then the
//     keys of the bin holding the k-th largest key (at most 64), whose
//     ranking gives the cut (the k-th selected key and column), then the
//     selected columns written in column order, staged in LDS and stored
//     in whole 1 KB blocks.  Rows of at most k candidates are copied.  A
//     row the bins do not settle is selected by 8-bit digits of its keys
//     (four counting reads) instead.
//   * Longer rows: one workgroup per row.  A 1/16 sample of the row (held in
//     registers) gives a threshold T below which the k-th largest key lies
//     only with a 4.5-sigma
//     miss of the sample; one pass lists every key >= T (about 1.4 k) in LDS
//     in column order, and the k-th largest listed key, the cut and the
//     selection come from the list.  A list with fewer than k keys or one
//     that overflows falls back to digit passes over the row (histograms of
//     the keys' top 11 bits, then of further digits of the chosen bin).
//   * With a workspace, at most 512 rows and rows longer than kSplitCols
//     (524288) columns, each such row is split over workgroups first: a
//     plan kernel orders the rows and sets each long row's key threshold
//     from a sample, a gather kernel lists the keys at or above it chunk by
//     chunk, and the selection works on the list (falling back as above when
//     the list is not whole or too short).
//
// The kernel is bound by instruction issue, not by HBM: eight wavefronts
// share a SIMD, and a row's latency is its per-tile instruction count times
// its passes.  So the hot loops keep selections in wavefront masks (a
// lane's bit used directly as a condition), test columns against the row's
// end only in the last round of tiles, store unconditionally (a spare slot
// per lane takes the columns not selected), and the rows that end last run
// at a raised instruction priority.
//
// Measured on MI355X (2048 rows of lognormal lengths up to 65536, k = 2048):
// the selection takes ~29 us per call, against ~59 us with one workgroup
// per row for every row; the groups of wavefronts hold the short and middle
// rows with little per-row overhead, while the long rows, a fifth of the
// rows but two thirds of the columns, get a workgroup each.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "pmqa_internal.h"

namespace pmqa {

namespace {

constexpr int kMaxSelWaves = 16;         // workgroups of 512 or 1024 threads
constexpr int kLoads = 8;                // 16-byte reads in flight per lane
constexpr int kTopBits = 11;             // first digit: key bits [21, 32)
constexpr int kTopShift = 32 - kTopBits;
constexpr int kBins = 1 << kTopBits;
constexpr int kCand = 1024;              // gathered keys of the chosen bin of a staged row
constexpr int kStage = 7680;             // rows up to this long are kept in LDS
constexpr int kCandLong = kStage / 2;    // ... of a longer row (in the unused stage; twice
                                         // that with 1024 threads)
constexpr int kBins2 = 256;              // later digits: at most 8 bits
constexpr int kWin = 4;                  // first-digit bins given a second digit in pass 1
constexpr int kSampleRun = 256;          // a row not in LDS is sampled: the first 256
constexpr int kSampleStride = 4096;      // columns of every 4096
constexpr int kListCap = kCandLong;      // keys listed for a split row, at most
constexpr int32_t kSplitCols = 65536 * 8;  // rows split with a workspace: longer than this
constexpr int kMaxChunks = 16;           // chunks of a split row, at most
constexpr int32_t kChunkMin = 16384;     // columns of a chunk, at least
constexpr int kRowSlots = 3 * kListCap / 2 + 32 * kMaxChunks;  // list slots of a row
constexpr uint32_t kNoSplit = 0xFFFFFFFFu;  // threshold of a row that is not split
constexpr int kPlanRun = 256;            // the plan samples 256 of every 4096 columns
constexpr float kListFill = 0.8f;        // expected list at most this share of kListCap

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// Larger value <-> larger key; -0 sorts just below +0.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Lanes below this one with their bit set in mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Candidates of row r: lengths[r] (clamped to [0, max_ctx]) when lengths is
// given, else the fused indexer rule: min(causal limit, 256 c_b, max_ctx)
// with c_b the row's unit count in the schedule (0 if the schedule header
// does not describe this call).
// Histogram adds of the digit passes, which count keys that may all be
// equal (a row of -inf past a context, a crowded digit): 64 same-address
// LDS atomics from one instruction are executed one after another, which
// made such a row of 65536 columns take over a millisecond.  When every
// lane of the wavefront adds to the first lane's bin (all four of a quad's
// columns, for hist_add4), one atomic adds them all; otherwise each adds
// its own.
__device__ __forceinline__ bool first_lane() {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(__builtin_amdgcn_read_exec() >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)__builtin_amdgcn_read_exec(),
                                                             0u)) == 0u;
}

__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)bin);
  const uint64_t exec = __builtin_amdgcn_read_exec();
  if (__builtin_amdgcn_ballot_w64(active & (bin == b0)) == exec) {  // uniform
    if (first_lane()) atomicAdd(&hist[b0], (uint32_t)__builtin_popcountll(exec));
  } else if (active) {
    atomicAdd(&hist[bin], 1u);
  }
}

__device__ __forceinline__ void hist_add4(uint32_t* hist, const uint32_t (&bin)[4],
                                          const bool (&active)[4]) {
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)bin[0]);
  bool all = true;
#pragma unroll
  for (int e = 0; e < 4; ++e) all = all & active[e] & (bin[e] == b0);
  const uint64_t exec = __builtin_amdgcn_read_exec();
  if (__builtin_amdgcn_ballot_w64(all) == exec) {  // uniform
    if (first_lane()) atomicAdd(&hist[b0], 4u * (uint32_t)__builtin_popcountll(exec));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (active[e]) atomicAdd(&hist[bin[e]], 1u);
  }
}

__device__ __forceinline__ int32_t row_candidates(int32_t r, int32_t max_ctx,
                                                  const int32_t* lengths, const int32_t* ctx,
                                                  const int32_t* sched, int32_t batch,
                                                  int32_t next_n, int32_t workers) {
  if (lengths) return min(max(lengths[r], 0), max_ctx);
  const int32_t b = r / next_n, j = r - b * next_n;
  const bool ok = sched[0] == kSchedMagic && sched[1] == batch && sched[2] == workers &&
                  sched[3] >= 0;
  const int32_t cap = (max_ctx + kUnit - 1) / kUnit;
  int32_t c = 0;
  if (ok) {
    const int32_t* S = sched + kSchedHeader + 2 * (workers + 1);
    c = min(max(S[b + 1] - S[b], 0), cap);
  }
  const int64_t lim = (int64_t)ctx[b] - next_n + 1 + j;
  return (int32_t)max((int64_t)0, min(min(lim, (int64_t)kUnit * c), (int64_t)max_ctx));
}

constexpr int kOrderBins = 128;           // count classes

// Columns of each chunk of a split row of n candidates: at least kChunkMin,
// and at most kMaxChunks chunks.
__device__ __forceinline__ int32_t chunk_cols(int32_t n) {
  const int64_t per = ((int64_t)n + kMaxChunks * 1024 - 1) / (kMaxChunks * 1024) * 1024;
  return (int32_t)(per > kChunkMin ? per : kChunkMin);
}

// First list slot of the chunk starting at column c of a row of n
// candidates (j chunks before it): each chunk gets 1.5 times its share of
// kListCap by columns, plus 32 (a chunk's count varies more, relative to its
// mean, the fewer keys it expects); kRowSlots for the row at most.
__device__ __forceinline__ int32_t chunk_slot(int32_t c, int32_t j, int32_t n) {
  return (int32_t)((int64_t)(3 * kListCap / 2) * c / n) + 32 * j;
}

// The workspace of the split path, in sections of whole 256-byte blocks.
struct SplitWs {
  int32_t* hdr;    // [0]: chunks listed
  int32_t* chunk;  // [rows * kMaxChunks]: (row << 4) | chunk, every chunk of every long row
  int32_t* map;    // [rows]: row taken by workgroup i of the selection
  int32_t* len;    // [rows]: candidates of each row
  uint32_t* thr;   // [rows]: key threshold of a split row, else kNoSplit
  int32_t* cnt;    // [rows * kMaxChunks]: keys at or above the threshold
  uint32_t* key;   // [rows * kRowSlots]: those keys, chunk by chunk (chunk_slot)
  int32_t* col;    // [rows * kRowSlots]: their columns
};

constexpr int64_t ws_words(int64_t n) { return (n + 63) & ~(int64_t)63; }

SplitWs split_ws(void* base, int32_t rows) {
  int32_t* p = static_cast<int32_t*>(base);
  SplitWs w;
  w.hdr = p;
  p += 64;
  w.chunk = p;
  p += ws_words((int64_t)rows * kMaxChunks);
  w.map = p;
  p += ws_words(rows);
  w.len = p;
  p += ws_words(rows);
  w.thr = reinterpret_cast<uint32_t*>(p);
  p += ws_words(rows);
  w.cnt = p;
  p += ws_words((int64_t)rows * kMaxChunks);
  w.key = reinterpret_cast<uint32_t*>(p);
  p += ws_words((int64_t)rows * kRowSlots);
  w.col = p;
  return w;
}

// Order-preserving coarse class of a candidate count: 0 for none, else
// 1 + 4 floor(log2 n) + the two bits below the leading one (at most 124).
__device__ __forceinline__ uint32_t count_class(int32_t n) {
  if (n <= 0) return 0;
  const int e = 31 - __builtin_clz((uint32_t)n);
  const int m = e >= 2 ? (n >> (e - 2)) & 3 : (e == 1 ? (n & 1) << 1 : 0);
  return 1u + 4u * (uint32_t)e + (uint32_t)m;
}

template <int kLong>
struct SelLdsT {
  union {
    uint32_t hist[kBins];        // pass 1
    struct {                     // after it
      uint32_t key[kCand];
      int32_t col[kCand];
    } cand;
  };
  uint32_t hist2[kBins2];
  union {
    float stage[kStage] __attribute__((aligned(16)));
    struct {
      uint32_t key[kLong];
      int32_t col[kLong];
    } cand_long;
  };
  uint32_t wave_gt[kMaxSelWaves], wave_eq[kMaxSelWaves], wave_sum[kMaxSelWaves];
  uint32_t cand_cnt[kMaxSelWaves];  // candidates each wavefront gathered
  int32_t chunk_cnt[kMaxChunks], chunk_lo[kMaxChunks];  // a split row's lists
  uint32_t chosen[3];  // bin, keys above it, keys in it
};

// Workgroups of 1024 threads (two per compute unit) have LDS for twice the
// gathered list of a long row.
template <int kSelThreads>
constexpr int long_cap() { return kSelThreads >= 1024 ? 2 * kCandLong : kCandLong; }
template <int kSelThreads>
using SelLds = SelLdsT<long_cap<kSelThreads>()>;

// Columns i..i+3 of a row, from LDS or global memory (two paths, so each
// compiles to its own load instructions), columns at or past c1 as -inf.
// Branch-free, so that several reads stay in flight: the quad read is the
// one at i clamped to the last quad holding a column below c1 (rows are
// allocated in whole quads: their stride is a multiple of 4), and the
// columns past c1 are masked afterwards.
template <class Lds>
__device__ __forceinline__ v4f load_cols(const float* row, const Lds& lds, bool staged,
                                         int32_t i, int32_t c1) {
  const float ninf = -__builtin_inff();
  const int32_t q = min(i, (c1 - 1) & ~3);
  v4f v = staged ? *reinterpret_cast<const v4f*>(lds.stage + q)
                 : *reinterpret_cast<const v4f*>(row + q);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = i + e < c1 ? v[e] : ninf;
  return v;
}

// The chunk [c0, c1) a wavefront owns, read 256 columns (4 per lane) per
// tile: calls f(first column of the lane's 4, values) for every tile in
// column order, kLoads tiles read ahead.
template <class Lds, class F>
__device__ __forceinline__ void for_each_tile(const float* row, const Lds& lds, bool staged,
                                              int32_t c0, int32_t c1, F&& f) {
  const int lane = threadIdx.x & 63;
  for (int32_t b0 = c0; b0 < c1; b0 += kLoads * 256) {
    v4f v[kLoads];
#pragma unroll
    for (int m = 0; m < kLoads; ++m)
      v[m] = load_cols(row, lds, staged, b0 + 256 * m + 4 * lane, c1);
#pragma unroll
    for (int m = 0; m < kLoads; ++m)
      if (b0 + 256 * m < c1) f(b0 + 256 * m + 4 * lane, v[m]);
  }
}

// The sample of a row not kept in LDS: the first kRun columns of every
// kSampleStride (so every read is part of a run of whole 1 KB lines);
// calls f(first column of the quad, values) for every quad of it.
template <int kSelThreads, int kRun, class Lds, class F>
__device__ __forceinline__ void for_each_sample(const float* row, const Lds& lds, int32_t n,
                                                F&& f) {
  constexpr int32_t kRunQuads = kRun / 4;
  const int32_t groups = (n + kSampleStride - 1) / kSampleStride;
  for (int32_t t = threadIdx.x; t < groups * kRunQuads; t += kSelThreads) {
    const int32_t col = kSampleStride * (t / kRunQuads) + 4 * (t % kRunQuads);
    if (col < n) f(col, load_cols(row, lds, false, col, n));
  }
}

template <int kRun>
__device__ __forceinline__ int32_t sample_size(int32_t n) {
  return kRun * (n / kSampleStride) + min(kRun, n % kSampleStride);
}

// Chooses the bin of hist[0..nbins) holding the krem-th largest key (bins
// counted from the top); every thread calls it.  Result in lds.chosen.
template <int kSelThreads, class Lds>
__device__ __forceinline__ void choose_bin(Lds& lds, const uint32_t* hist, int nbins,
                                           uint32_t krem) {
  const int per = (nbins + kSelThreads - 1) / kSelThreads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bhi = nbins - 1 - per * tid;
  uint32_t own = 0;
  for (int j = 0; j < per; ++j)
    if (bhi - j >= 0) own += hist[bhi - j];
  uint32_t incl = own;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) lds.wave_sum[wave] = incl;
  __syncthreads();
  uint32_t above = incl - own;
  for (int w = 0; w < wave; ++w) above += lds.wave_sum[w];
  for (int j = 0; j < per; ++j) {
    if (bhi - j < 0) break;
    const uint32_t h = hist[bhi - j];
    if (above < krem && krem <= above + h) {
      lds.chosen[0] = (uint32_t)(bhi - j);
      lds.chosen[1] = above;
      lds.chosen[2] = h;
    }
    above += h;
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// ---- value-linear bins and the listing path of a long row
//
// Values are binned linearly over a range [lo, hi]: bin(x) = clamp((x - lo)
// s, 0, kFastBins - 1) truncated, s = kFastBins / (hi - lo).  Every step of
// that map is monotone (a rounded subtraction and product, a clamp, a
// truncation), so a key in a lower bin is never larger than a key in a
// higher one, whatever the rounding; values outside [lo, hi] land in the end
// bins.  Unlike bins of the keys' top bits, where most of a row's values
// share the sign and exponent and crowd into a few bins, it spreads a row's
// values over all bins.  Once the bin b of the k-th largest key is known,
// its keys (at most 64) are listed in LDS and ranked, (key, column) against
// (key, column); that gives the cut: the k-th selected key K and column C,
// so that a column is selected exactly when its key is above K, or equal to
// K at a column <= C.
//
// A long row's workgroup samples it (256 of every 4096 columns); the
// sample's bins give a value T below which the k-th largest key lies only
// with a 4.5-sigma miss of the sample, and about 1.4 k keys are expected at
// or above it.  One pass lists every key >= T in LDS, in column order, each
// wavefront in its own region; the k-th largest listed key is found with a
// histogram of the list as above (its top bin bounded by the sample's
// largest value), and the selection is written from the list.  A list with
// fewer than k keys, a region that overflows or more than 64 keys in the
// chosen bin sends the row to the digit passes, with the same result.
constexpr int kFastBins = 1024;
constexpr int kSmall = 64;     // keys of the k-th key's bin, at most
constexpr int kListLoads = 8;  // 16-byte reads in flight per lane in the listing pass

template <int kSelThreads>
constexpr int fast_cap() { return kSelThreads >= 1024 ? 10240 : 5120; }

template <int kSelThreads>
struct FastLds {
  static constexpr int kW = kSelThreads / 64;
  uint32_t hist[kFastBins + 4];
  uint32_t hist2[kFastBins + 4];
  float key[fast_cap<kSelThreads>()];      // listed keys (their values), per-wavefront regions
  uint16_t col[fast_cap<kSelThreads>()];   // their columns, from the wavefront's first
  uint32_t skey[kSmall];                   // the keys of bin b ...
  int32_t scol[kSmall];                    // ... and their columns
  float wlo[kW], whi[kW];
  uint32_t wcnt[kW];
  uint32_t scnt;
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// A wavefront's chunk [c0, c1) of a row as a buffer resource (whole quads:
// a row's storage extends to a multiple of 4 columns); a read past it
// returns zeros without touching memory.
__device__ __forceinline__ rsrc_t chunk_rsrc(const float* row, int32_t c0, int32_t c1) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row + c0), 0,
                                           ((c1 - c0 + 3) & ~3) * 4, 0x00020000);
}

// Columns t + 4 lane .. + 3 of a chunk (t from the chunk's first column), as
// stored: the caller masks the columns past the chunk's end.
__device__ __forceinline__ v4f rload(rsrc_t rs, int32_t t, int lane) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 4 * t, 0));
}

// Columns col..col+3 of a row of n candidates from global memory (the quad
// read is clamped to the row's last quad), those at or past n as -inf.
__device__ __forceinline__ v4f quad_at(const float* row, int32_t col, int32_t n) {
  const float ninf = -__builtin_inff();
  v4f v = *reinterpret_cast<const v4f*>(row + min(col, (n - 1) & ~3));
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = col + e < n ? v[e] : ninf;
  return v;
}

// The sample of a long row (the listing path): G runs of 256 columns, one
// per 4096 columns of the row up to two quads per thread (G at most
// 2 kSelThreads / 64), run g starting at column g D, D = floor(n / G)
// rounded down to a multiple of 4: runs at least 3072 columns apart for
// rows of more than 6144, the last ending at most n - D + 256 < n.  Quad q
// of the sample (of 64 G) is read by thread q mod kSelThreads.
template <int kSelThreads>
__device__ __forceinline__ int32_t sample_runs(int32_t n) {
  return min((n + 4095) / 4096, 2 * kSelThreads / 64);
}

__device__ __forceinline__ uint32_t lin_bin(float x, float lo, float s) {
  return (uint32_t)__builtin_amdgcn_fmed3f((x - lo) * s, 0.f, (float)(kFastBins - 1));
}

// Inclusive scan over the wavefront's 64 lanes with DPP: shifts within rows
// of 16 lanes (row_shr 1, 2, 4, 8), then the last lane of row 0 into row 1
// and of row 2 into row 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31).  A lane without a source takes `id`.  No lane-address
// registers are needed, unlike permute-based shuffles.
template <class F>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, F op) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}

// Wavefront-wide minimum / maximum (uniform results).
__device__ __forceinline__ float wave_min(float x) {
  const uint32_t r = wave_scan(__float_as_uint(x), __float_as_uint(__builtin_inff()),
                               [](uint32_t a, uint32_t b) {
                                 return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
                               });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
}
__device__ __forceinline__ float wave_max(float x) {
  const uint32_t r = wave_scan(__float_as_uint(x), __float_as_uint(-__builtin_inff()),
                               [](uint32_t a, uint32_t b) {
                                 return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
                               });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
}

__device__ __forceinline__ uint32_t scan_add(uint32_t x) {
  return wave_scan(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive scans within each row of 16 lanes (DPP row shifts).
__device__ __forceinline__ uint32_t row16_scan_add(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
  return x;
}

template <int NB = kFastBins>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t r, uint32_t& bin,
                                         uint32_t& above, uint32_t& h) {
  constexpr int kPer = NB / 64;
  static_assert(kPer == 16 || kPer == 4, "16 or 4 bins per lane");
  const int lane = threadIdx.x & 63;
  const int base = NB - kPer * (lane + 1);
  uint32_t own = 0;
  const uint4* p = reinterpret_cast<const uint4*>(hist + base);
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {
    const uint4 u = p[q];
    own += u.x + u.y + u.z + u.w;
  }
  const uint32_t incl = scan_add(own);
  const uint32_t excl = incl - own;
  const uint64_t m = __ballot(excl < r && r <= incl);
  const int src = m ? __builtin_ctzll(m) : 0;
  const uint32_t ex = (uint32_t)__builtin_amdgcn_readlane((int)excl, src);
  const int jb = NB - kPer * src - 1 - (lane & (kPer - 1));  // lane j of a row: the j-th bin from the top
  const uint32_t c = hist[jb];
  const uint32_t ic = ex + row16_scan_add(c);
  const uint64_t m2 = __ballot(lane < kPer && ic - c < r && r <= ic);
  const int s2 = m2 ? __builtin_ctzll(m2) : 0;
  bin = (uint32_t)__builtin_amdgcn_readlane(jb, s2);
  above = (uint32_t)__builtin_amdgcn_readlane((int)(ic - c), s2);
  h = (uint32_t)__builtin_amdgcn_readlane((int)c, s2);
}

// The cut: the krem-th of the h keys of bin b (h <= kSmall, listed in LDS)
// in the order (key descending, column ascending); every wavefront computes
// it alone, lane j ranking key j against the others read lane by lane.  Also
// returns how many of the bin's selected keys lie before column c0.
__device__ __forceinline__ void find_cut(const uint32_t* skey, const int32_t* scol, uint32_t h,
                                         uint32_t krem, int32_t c0, uint32_t& kc,
                                         int32_t& cc, uint32_t& before) {
  const int lane = threadIdx.x & 63;
  const bool in = (uint32_t)lane < h;
  const uint32_t kj = in ? skey[lane] : 0u;
  const int32_t cj = in ? scol[lane] : 0;
  uint32_t rank = 0;
  for (uint32_t i = 0; i < h; ++i) {
    const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, (int)i);
    const int32_t ci = __builtin_amdgcn_readlane(cj, (int)i);
    rank += ((ki > kj) | ((ki == kj) & (ci < cj))) ? 1u : 0u;
  }
  const uint64_t mc = __ballot(in & (rank + 1 == krem));
  const int src = mc ? __builtin_ctzll(mc) : 0;
  kc = (uint32_t)__builtin_amdgcn_readlane((int)kj, src);
  cc = __builtin_amdgcn_readlane(cj, src);
  before = (uint32_t)__builtin_popcountll(__ballot(in & (rank < krem) & (cj < c0)));
}

template <int kSelThreads>
__device__ __forceinline__ bool fast_list(FastLds<kSelThreads>& f, const float* row, int32_t n,
                                          int32_t k, int32_t* oi, float* ov) {
  constexpr int W = kSelThreads / 64;
  constexpr uint32_t R = (uint32_t)fast_cap<kSelThreads>() / W;  // entries of a region
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t L = ((n + W - 1) / W + 3) & ~3;
  if (L > 65536) return false;  // column offsets are 16-bit; no LDS touched yet
  const int32_t c0 = min(n, wave * L), c1 = min(n, c0 + L);
  for (int j = tid; j <= kFastBins; j += kSelThreads) {
    f.hist[j] = 0u;
    f.hist2[j] = 0u;
  }
  if (tid == 0) f.scnt = 0u;
  // 1. The sample (held in registers: quads tid and tid + kSelThreads), its
  //    range, then its histogram.  (Issuing the listing's first reads here
  //    too, to arrive while the sample is counted, measured no faster: the
  //    sample's own reads then took as much longer.)
  const int32_t G = sample_runs<kSelThreads>(n), nq = 64 * G;
  const int32_t D = __builtin_amdgcn_readfirstlane((n / G) & ~3);
  const bool in0 = tid < nq, in1 = tid + kSelThreads < nq;
  const int32_t q0 = in0 ? tid : 0, q1 = in1 ? tid + kSelThreads : 0;
  const v4f s0 = *reinterpret_cast<const v4f*>(row + (q0 >> 6) * D + 4 * (q0 & 63));
  const v4f s1 = *reinterpret_cast<const v4f*>(row + (q1 >> 6) * D + 4 * (q1 & 63));
  float lo = __builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (in0 & __builtin_isfinite(s0[e])) {
      lo = fminf(lo, s0[e]);
      hi = fmaxf(hi, s0[e]);
    }
    if (in1 & __builtin_isfinite(s1[e])) {
      lo = fminf(lo, s1[e]);
      hi = fmaxf(hi, s1[e]);
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    f.wlo[wave] = lo;
    f.whi[wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < W; ++w) {
    lo = fminf(lo, f.wlo[w]);
    hi = fmaxf(hi, f.whi[w]);
  }
  const float s = (float)kFastBins * __builtin_amdgcn_rcpf(hi - lo);
  if (!(hi > lo) || !(s > 0.f) || !__builtin_isfinite(s)) {
    __syncthreads();
    return false;
  }
  {
    // values below the sample's finite range (a row of -inf past its
    // context) all land in bin 0: a wavefront of them adds with one atomic
    uint32_t b0[4], b1[4];
    bool a0[4], a1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b0[e] = lin_bin(s0[e], lo, s);
      b1[e] = lin_bin(s1[e], lo, s);
      a0[e] = in0;
      a1[e] = in1;
    }
    hist_add4(f.hist, b0, a0);
    hist_add4(f.hist, b1, a1);
  }
  __syncthreads();
  // T: one bin below the sample key of rank ks + 4.5 sqrt(ks) + 4.5
  const int32_t ns = 256 * G;
  const float ks = (float)k * (float)ns / (float)n;
  const uint32_t rs = (uint32_t)min((float)ns, ceilf(ks + 4.5f * sqrtf(ks) + 4.5f));
  uint32_t bs, a0, h0;
  find_bin<>(f.hist, rs, bs, a0, h0);
  const float T = lo + ((float)bs - 1.f) * ((hi - lo) * (1.f / (float)kFastBins));
  // 2. Every key >= T, in column order, into the wavefront's region: a
  //    ring of kListLoads tiles in flight, each slot refilled (kListLoads
  //    tiles ahead) as soon as it is used; reads past the chunk touch no
  //    memory.
  const rsrc_t rs_c = chunk_rsrc(row, c0, c1);
  float* lkey = f.key + wave * R;
  uint16_t* lcol = f.col + wave * R;
  uint32_t mine = 0;
  v4f x[kListLoads];
#pragma unroll
  for (int m = 0; m < kListLoads; ++m) x[m] = rload(rs_c, 256 * m, lane);
  // A tile's keys are listed only while the region has room for them and,
  // past them, for a slot per lane that takes the stores of the lane's keys
  // not listed (rewritten later, or never read), so that every store is
  // unconditional; a tile without that room marks the region as overflowed
  // (the row then takes the digit passes).
  auto list_tile = [&](const v4f& v, int32_t t, const uint64_t (&ms)[4]) {
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) tot += (uint32_t)__builtin_popcountll(ms[e]);
    if (mine + tot + 64u <= R) {
      uint32_t slot = mine;
#pragma unroll
      for (int e = 0; e < 4; ++e) slot += lanes_below(ms[e]);
      const uint32_t spare = mine + tot + (uint32_t)lane;
      const uint32_t off = (uint32_t)(t + 4 * lane - c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = __builtin_amdgcn_inverse_ballot_w64(ms[e]);
        const uint32_t q = in ? slot : spare;
        lkey[q] = v[e];
        lcol[q] = (uint16_t)(off + e);
        slot += in ? 1u : 0u;
      }
      mine += tot;
    } else {
      mine = R + 1u;
    }
  };
  // rounds of kListLoads whole tiles, then the chunk's last, partial round
  // (the loop's last refills read past the chunk: zeros, no memory touched)
  int32_t b0 = c0;
  for (; b0 + kListLoads * 256 <= c1; b0 += kListLoads * 256) {  // uniform
#pragma unroll
    for (int m = 0; m < kListLoads; ++m) {
      uint64_t ms[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ms[e] = __builtin_amdgcn_ballot_w64(x[m][e] >= T);
      list_tile(x[m], b0 + 256 * m, ms);
      x[m] = rload(rs_c, b0 - c0 + 256 * (m + kListLoads), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int m = 0; m < kListLoads; ++m) {
    const int32_t t = b0 + 256 * m;  // uniform
    uint64_t ms[4];
    if (t + 256 <= c1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ms[e] = __builtin_amdgcn_ballot_w64(x[m][e] >= T);
      list_tile(x[m], t, ms);
    } else if (t < c1) {
      // columns of the lane at or past c1 (the chunk's end) are not the row's
      const int32_t lim = c1 - (t + 4 * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) ms[e] = __builtin_amdgcn_ballot_w64((x[m][e] >= T) & (e < lim));
      list_tile(x[m], t, ms);
    }
  }
  if (lane == 0) f.wcnt[wave] = mine;
  __syncthreads();
  uint32_t total = 0;
  bool over = false;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    total += f.wcnt[w];
    over = over || f.wcnt[w] > R;
  }
  // 3. The k-th largest listed key: bins over [T, sample max].  The
  //    wavefront's listed keys and their bins stay in registers for the
  //    rest of the row (all of the region's reads issued at once): no
  //    dependent LDS reads per round of 64 keys.
  const float s2 = hi > T ? (float)kFastBins * __builtin_amdgcn_rcpf(hi - T) : 0.f;
  if (over || total < (uint32_t)k || !(s2 > 0.f) || !__builtin_isfinite(s2)) {
    __syncthreads();
    return false;
  }
  constexpr int kT = (int)(R + 63) / 64;
  const uint32_t nt = (mine + 63) / 64;  // rounds of 64 keys the wavefront listed (uniform)
  float kv[kT];
  uint32_t bn[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t)
    if (t < nt) kv[t] = 64u * t + lane < mine ? lkey[64 * t + lane] : T;  // slots past `mine` hold no key
#pragma unroll
  for (int t = 0; t < kT; ++t)
    if (t < nt) {
      bn[t] = lin_bin(kv[t], T, s2);
      if (64u * t + lane < mine) atomicAdd(&f.hist2[bn[t]], 1u);
    }
  __syncthreads();
  uint32_t b, above, h;
  find_bin<>(f.hist2, (uint32_t)k, b, above, h);
  if (h > kSmall) {
    __syncthreads();
    return false;
  }
  uint32_t gt = 0;
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    if (t >= nt) break;  // uniform
    const bool in = 64u * t + lane < mine;
    gt += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(in & (bn[t] > b)));
    if (in & (bn[t] == b)) {
      const uint32_t slot = atomicAdd(&f.scnt, 1u);
      if (slot < (uint32_t)kSmall) {
        f.skey[slot] = order_key(kv[t]);
        f.scol[slot] = c0 + (int32_t)lcol[64 * t + lane];
      }
    }
  }
  if (lane == 0) f.wcnt[wave] = gt;  // every wavefront read the counts above before the last barrier
  __syncthreads();
  uint32_t kc, pos;
  int32_t cc;
  find_cut(f.skey, f.scol, h, (uint32_t)k - above, c0, kc, cc, pos);
#pragma unroll
  for (int w = 0; w < W; ++w) pos += w < wave ? f.wcnt[w] : 0u;
  // 4. The selection, from the wavefront's region in order.
  int32_t col[kT];
#pragma unroll
  for (int t = 0; t < kT; ++t)
    if (t < nt) col[t] = c0 + (int32_t)lcol[64 * t + lane];
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    if (t >= nt) break;  // uniform
    const bool in = 64u * t + lane < mine;
    const uint32_t key = order_key(kv[t]);
    const bool sel = in & ((key > kc) | ((key == kc) & (col[t] <= cc)));
    const uint64_t m = __builtin_amdgcn_ballot_w64(sel);
    const uint32_t p = pos + lanes_below(m);
    if (sel & (p < (uint32_t)k)) {
      oi[p] = col[t];
      if (ov) ov[p] = kv[t];
    }
    pos += (uint32_t)__builtin_popcountll(m);
  }
  return true;
}

// ---- one wavefront per row
//
// A row of at most kWaveCols candidates is selected by one wavefront alone,
// with no workgroup barrier: eight such rows share a workgroup (one per
// wavefront), while longer rows get a workgroup each.  The wavefront reads
// its row three times (the first read from HBM, the others mostly from the
// caches), 256 columns per read instruction and kRing reads in flight:
//   1. value-linear bins over the range of a 64-point sample of the row
//      (values outside it land in the end bins), counted in the
//      wavefront's own histogram;
//   2. the keys of the bin b of the k-th largest key (at most 64) listed with
//      their columns, and the cut found from them;
//   3. the selected columns in column order, each lane's rank within the
//      wavefront from ballots, staged in LDS and written in whole blocks.
// A row whose sample has no finite range or whose bin b holds more than 64
// keys is selected by 8-bit digits of its keys instead (four counting reads
// and the write), the k-th key's equal keys taken by column.
constexpr int32_t kWaveCols = 6144;  // rows selected by one wavefront, at most
constexpr int kRing = 4;             // 16-byte reads in flight per lane

constexpr int kOutSlots = 512 + 64;  // staging slots: two blocks of 256, then one per lane

struct alignas(16) WaveLds {
  union {
    uint32_t hist[kFastBins + 4];  // [kFastBins]: columns out of range
    struct {
      int32_t idx[kOutSlots];
      float val[kOutSlots];
    } out;  // the write's staging, once the histogram is no longer read
  };
  uint32_t skey[kSmall];
  int32_t scol[kSmall];
};

// Columns t + 4 lane .. + 3 of a row through its buffer resource (reads past
// the row's storage return zeros without touching memory).
__device__ __forceinline__ v4f row_quad(rsrc_t rs, int32_t t, int lane) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 4 * t, 0));
}

template <bool B>
struct Whole {
  static constexpr bool value = B;
};

// Calls f(first column of the lane's quad, values, Whole<w>) for every tile
// of 256 columns of the row in order, kRing reads in flight: each slot of
// the ring is refilled kRing tiles ahead right after its tile is used.  The
// loop takes the rounds of kRing tiles whose columns are all the row's
// (w true: no column needs a test); the row's last, partial round follows
// it (w false), with no further reads (reads past the row return zeros
// without touching memory, so the loop's last refills are harmless).
template <class F>
__device__ __forceinline__ void each_tile(rsrc_t rs, int32_t n, F&& f) {
  const int lane = threadIdx.x & 63;
  v4f x[kRing];
#pragma unroll
  for (int m = 0; m < kRing; ++m) x[m] = row_quad(rs, 256 * m, lane);
  int32_t t0 = 0;
  for (; t0 + kRing * 256 <= n; t0 += kRing * 256) {  // uniform
#pragma unroll
    for (int m = 0; m < kRing; ++m) {
      f(t0 + 256 * m + 4 * lane, x[m], Whole<true>{});
      x[m] = row_quad(rs, t0 + 256 * (m + kRing), lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int m = 0; m < kRing; ++m)
    if (t0 + 256 * m < n) f(t0 + 256 * m + 4 * lane, x[m], Whole<false>{});
}

// The selection of a row leaves through LDS: output entry p goes to slot
// p mod 512 (two blocks of 256), and a block, once whole, is written with
// one 16-byte store per lane for the indices and one for the values (1 KB
// of consecutive output per instruction).  Written where they are ranked,
// the entries would go out as 4-byte stores scattered over partial lines:
// 33.6 MB of output took 16.4 us that way on MI355X, 7.4 us in 16-byte
// stores.  `vec`: both output rows are 16-byte aligned; else a block leaves
// as 4-byte stores, 256 consecutive bytes per instruction.
__device__ __forceinline__ void flush_block(const WaveLds& w, uint32_t j, uint32_t cnt,
                                            int32_t* oi, float* ov, bool vec) {
  const int lane = threadIdx.x & 63;
  const uint32_t s = (j & 1u) * 256u, p = 256u * j;
  __builtin_amdgcn_wave_barrier();
  if (vec & (cnt == 256u)) {
    const v4i a = *reinterpret_cast<const v4i*>(w.out.idx + s + 4 * lane);
    *reinterpret_cast<v4i*>(oi + p + 4 * lane) = a;
    if (ov) {
      const v4f v = *reinterpret_cast<const v4f*>(w.out.val + s + 4 * lane);
      *reinterpret_cast<v4f*>(ov + p + 4 * lane) = v;
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t e = 64u * m + (uint32_t)lane;
      if (e < cnt) {
        oi[p + e] = w.out.idx[s + e];
        if (ov) ov[p + e] = w.out.val[s + e];
      }
    }
  }
}

// Stages the lane's selected columns of one quad (bit `lane` of ms[e]:
// column i + e) at their ranks, pos plus the selected columns of the lower
// lanes and of the lane's own lower columns, and writes out the block the
// quad completes, if any (a quad adds at most 256 entries, so at most one).
// Every lane stores all four columns, those not selected into the lane's
// own slot past the blocks, so no store waits on a branch.  A row selects
// exactly k columns (fewer or more only for a row holding NaN, whose
// selection is unspecified: every store stays in the staging).  The
// selection stays in wavefront masks (scalar registers) throughout; a
// lane's bit is used as a condition directly (inverse ballot).
__device__ __forceinline__ void stage_quad(WaveLds& w, const v4f& x, int32_t i,
                                           const uint64_t (&ms)[4], uint32_t& pos, int32_t k,
                                           int32_t* oi, float* ov, bool vec) {
  const int lane = threadIdx.x & 63;
  uint32_t p = pos;
#pragma unroll
  for (int e = 0; e < 4; ++e) p += lanes_below(ms[e]);
  const uint32_t trash = 512u + (uint32_t)lane;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool in = __builtin_amdgcn_inverse_ballot_w64(ms[e]);
    const uint32_t q = in ? (p & 511u) : trash;
    w.out.idx[q] = i + e;
    w.out.val[q] = x[e];
    p += in ? 1u : 0u;
  }
  uint32_t tot = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) tot += (uint32_t)__builtin_popcountll(ms[e]);
  const uint32_t before = min(pos, (uint32_t)k) >> 8, after = min(pos + tot, (uint32_t)k) >> 8;
  if (after != before) flush_block(w, before, 256u, oi, ov, vec);
  pos += tot;
}

// Writes the last, partial block of a row of k selected entries.
__device__ __forceinline__ void finish_rows(const WaveLds& w, int32_t k, int32_t* oi, float* ov,
                                            bool vec) {
  if (k & 255) flush_block(w, (uint32_t)k >> 8, (uint32_t)k & 255u, oi, ov, vec);
}

__device__ __forceinline__ bool aligned16(const int32_t* oi, const float* ov) {
  return ((reinterpret_cast<uintptr_t>(oi) | reinterpret_cast<uintptr_t>(ov)) & 15u) == 0;
}

// The value of an order key (the inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// A wavefront row's bins: value-linear over the sample's range like lin_bin,
// as one fused multiply-add (x s - lo s), a clamp and a truncation: monotone
// in x, like every step.
__device__ __forceinline__ uint32_t fast_bin(float x, float s, float c) {
  return (uint32_t)__builtin_amdgcn_fmed3f(__builtin_fmaf(x, s, c), 0.f, (float)(kFastBins - 1));
}

__device__ __forceinline__ bool wave_fast(WaveLds& w, const float* row, rsrc_t rs, int32_t n,
                                          int32_t k, int32_t* oi, float* ov) {
  const int lane = threadIdx.x & 63;
  // the range of a sample of 64 columns spread over the row
  const float sv = row[(int32_t)(((int64_t)lane * n) >> 6)];
  for (int j = lane; j <= kFastBins; j += 64) w.hist[j] = 0u;
  const float lo = wave_min(sv), hi = wave_max(sv);
  const float s = (float)kFastBins * __builtin_amdgcn_rcpf(hi - lo);
  if (!(hi > lo) || !(s > 0.f) || !__builtin_isfinite(s)) return false;
  const float c = -lo * s;
  // 1. the histogram (columns past n go to the extra bin)
  each_tile(rs, n, [&](int32_t i, const v4f& x, auto whole) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t bin = fast_bin(x[e], s, c);
      if (!decltype(whole)::value) bin = i + e < n ? bin : (uint32_t)kFastBins;
      atomicAdd(&w.hist[bin], 1u);
    }
  });
  uint32_t b, above, h;
  find_bin<>(w.hist, (uint32_t)k, b, above, h);
  if (h > kSmall) return false;
  // 2. the keys of bin b (a few tiles hold any), then the cut
  uint32_t listed = 0;
  each_tile(rs, n, [&](int32_t i, const v4f& x, auto whole) {
    uint64_t ms[4], any = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool in = fast_bin(x[e], s, c) == b;
      if (!decltype(whole)::value) in = in & (i + e < n);
      ms[e] = __builtin_amdgcn_ballot_w64(in);
      any |= ms[e];
    }
    if (any) {
      uint32_t slot = listed;
#pragma unroll
      for (int e = 0; e < 4; ++e) slot += lanes_below(ms[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = __builtin_amdgcn_inverse_ballot_w64(ms[e]);
        if (in & (slot < (uint32_t)kSmall)) {
          w.skey[slot] = order_key(x[e]);
          w.scol[slot] = i + e;
        }
        slot += in ? 1u : 0u;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) listed += (uint32_t)__builtin_popcountll(ms[e]);
    }
  });
  uint32_t kc, unused;
  int32_t cc;
  find_cut(w.skey, w.scol, h, (uint32_t)k - above, 0, kc, cc, unused);
  // 3. the selection (exactly k columns): a key above the cut's, or equal
  //    to it at a column <= cc.  Where the cut's value is a normal float
  //    with a normal float just below it, a key is above the cut's exactly
  //    when its value is above the cut value, and equal or above exactly
  //    when above that lower float: one compare per column, against a
  //    threshold chosen by the column.  Otherwise (zeros, whose keys differ
  //    but whose values compare equal; denormals; infinities) the keys are
  //    compared.
  const bool vec = aligned16(oi, ov);
  const float xc = key_value(kc);
  const uint32_t xb = __float_as_uint(xc);
  const uint32_t ex = (xb >> 23) & 0xFFu;
  uint32_t pos = 0;
  if ((ex >= 2u) & (ex <= 254u)) {
    const float xlo = __uint_as_float((xb & 0x80000000u) ? xb + 1u : xb - 1u);
    each_tile(rs, n, [&](int32_t i, const v4f& x, auto whole) {
      uint64_t ms[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool sel = x[e] > (i + e <= cc ? xlo : xc);
        if (!decltype(whole)::value) sel = sel & (i + e < n);
        ms[e] = __builtin_amdgcn_ballot_w64(sel);
      }
      stage_quad(w, x, i, ms, pos, k, oi, ov, vec);
    });
  } else {
    each_tile(rs, n, [&](int32_t i, const v4f& x, auto whole) {
      uint64_t ms[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = order_key(x[e]);
        bool sel = (key > kc) | ((key == kc) & (i + e <= cc));
        if (!decltype(whole)::value) sel = sel & (i + e < n);
        ms[e] = __builtin_amdgcn_ballot_w64(sel);
      }
      stage_quad(w, x, i, ms, pos, k, oi, ov, vec);
    });
  }
  finish_rows(w, k, oi, ov, vec);
  return true;
}

// The k-th largest key by 8-bit digits (four counting reads), then the
// write: keys above it, and its equal keys in column order while they last.
__device__ __forceinline__ void wave_radix(WaveLds& w, rsrc_t rs, int32_t n, int32_t k,
                                           int32_t* oi, float* ov) {
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
  for (int d = 24; d >= 0; d -= 8) {
    const int lane = threadIdx.x & 63;
    for (int j = lane; j < 256; j += 64) w.hist[j] = 0u;
    each_tile(rs, n, [&](int32_t i, const v4f& x, auto) {
      uint32_t bin[4];
      bool act[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = order_key(x[e]);
        bin[e] = (key >> d) & 0xFFu;
        act[e] = (i + e < n) & ((key & pmask) == prefix);
      }
      hist_add4(w.hist, bin, act);
    });
    uint32_t g, above, h;
    find_bin<256>(w.hist, krem, g, above, h);
    prefix |= g << d;
    pmask |= 0xFFu << d;
    krem -= above;
  }
  // prefix is the k-th largest key; krem of its equal keys are taken (k
  // columns in all)
  const bool vec = aligned16(oi, ov);
  uint32_t pos = 0, eq = 0;
  each_tile(rs, n, [&](int32_t i, const v4f& x, auto) {
    bool isq[4];
    uint64_t mq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      isq[e] = (i + e < n) & (order_key(x[e]) == prefix);
      mq[e] = __ballot(isq[e]);
    }
    uint32_t r = eq;  // equal keys before this lane's first column
#pragma unroll
    for (int e = 0; e < 4; ++e) r += lanes_below(mq[e]);
    uint64_t ms[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ms[e] = __builtin_amdgcn_ballot_w64(((i + e < n) & (order_key(x[e]) > prefix)) |
                                          (isq[e] & (r < krem)));
      r += isq[e] ? 1u : 0u;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) eq += (uint32_t)__builtin_popcountll(mq[e]);
    stage_quad(w, x, i, ms, pos, k, oi, ov, vec);
  });
  finish_rows(w, k, oi, ov, vec);
}

// One row by one wavefront.
__device__ __forceinline__ void select_row_wave(WaveLds& w, const float* row, int32_t n, int32_t k,
                                                int32_t* oi, float* ov) {
  const int lane = threadIdx.x & 63;
  if (n <= k) {  // every candidate is selected: 4 columns per lane, 4 reads in flight
    const float ninf = -__builtin_inff();
    const bool vec = aligned16(oi, ov);
    for (int32_t i0 = 4 * lane; i0 < k; i0 += 4 * 256) {
      v4f x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int32_t i = i0 + 256 * m;  // a quad of the row's storage when i < n
        x[m] = i < n ? *reinterpret_cast<const v4f*>(row + i) : v4f{ninf, ninf, ninf, ninf};
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int32_t i = i0 + 256 * m;
        v4i a;
        v4f v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = i + e < n ? i + e : -1;
          v[e] = i + e < n ? x[m][e] : ninf;
        }
        if (vec & (i + 3 < k)) {  // whole quads in 16-byte stores
          *reinterpret_cast<v4i*>(oi + i) = a;
          if (ov) *reinterpret_cast<v4f*>(ov + i) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (i + e < k) {
              oi[i + e] = a[e];
              if (ov) ov[i + e] = v[e];
            }
        }
      }
    }
    return;
  }
  const rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0,
                                                      ((n + 3) & ~3) * 4, 0x00020000);
  if (!wave_fast(w, row, rs, n, k, oi, ov)) wave_radix(w, rs, n, k, oi, ov);
}

// The selection of one row by the whole workgroup: a row of at most k
// candidates is copied; a split row's list is used when whole; a row held in
// registers or a longer row takes its fast path; anything else (or a fast
// path that cannot settle the row) takes the digit passes.
template <int kSelThreads>
__device__ __forceinline__ void select_row_wg(SelLds<kSelThreads>& lds, FastLds<kSelThreads>& fast,
                                              const float* row, int64_t r, int32_t n, int32_t k,
                                              int32_t* oi, float* ov, SplitWs ws) {
  constexpr int kSelWaves = kSelThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float ninf = -__builtin_inff();

  if (n <= k) {  // every candidate is selected
    for (int32_t i = tid; i < k; i += kSelThreads) {
      oi[i] = i < n ? i : -1;
      if (ov) ov[i] = i < n ? row[i] : ninf;
    }
    return;
  }

  const int32_t L = ((n + kSelWaves - 1) / kSelWaves + 3) & ~3;
  const int32_t c0 = min(n, wave * L), c1 = min(n, c0 + L);
  const bool staged = n <= kStage;

  // Resolves the key bits under `top` of the k-th largest key among the
  // gathered keys matching prefix under pmask (krem-th of those); digits of
  // `bits` bits counted in hist (1 << bits bins), every thread calls it.
  // Slots from `limit` on hold no key.
  auto resolve = [&](uint32_t* ckey, uint32_t R, int top, uint32_t& pmask, uint32_t& prefix,
                     uint32_t& krem, int bits = 8, uint32_t* hist = nullptr,
                     uint32_t limit = 0xFFFFFFFFu) {
    if (!hist) hist = lds.hist2;
    limit = min(limit, R * kSelWaves);
    while (top > 0) {
      const int shift = max(top - bits, 0);
      const uint32_t dmask = (1u << (top - shift)) - 1u;
      for (int b = tid; b <= (int)dmask; b += kSelThreads) hist[b] = 0;
      __syncthreads();
      for (uint32_t c = tid; c < limit; c += kSelThreads) {
        const uint32_t key = ckey[c];
        hist_add(hist, (key >> shift) & dmask,
                 (c % R < lds.cand_cnt[c / R]) & ((key & pmask) == prefix));
      }
      __syncthreads();
      choose_bin<kSelThreads>(lds, hist, (int)dmask + 1, krem);
      prefix |= lds.chosen[0] << shift;
      pmask |= dmask << shift;
      krem -= lds.chosen[1];
      const uint32_t h = lds.chosen[2];
      __syncthreads();
      top = shift;
      if (top > 0 && h <= 64) {
        // at most 64 keys share the prefix: one wavefront ranks them
        uint32_t* small = lds.hist2;  // keys [0, 64), count at [64]
        if (tid == 0) small[64] = 0;
        __syncthreads();
        for (uint32_t c = tid; c < limit; c += kSelThreads) {
          const uint32_t key = ckey[c];
          if (c % R < lds.cand_cnt[c / R] && (key & pmask) == prefix)
            small[atomicAdd(&small[64], 1u)] = key;
        }
        __syncthreads();
        if (wave == 0) {
          const uint32_t cnt = small[64];
          const uint32_t mine = lane < (int)cnt ? small[lane] : 0u;
          uint32_t gt = 0, ge = 0;
          for (uint32_t j = 0; j < cnt; ++j) {
            const uint32_t o = small[j];
            gt += o > mine ? 1u : 0u;
            ge += o >= mine ? 1u : 0u;
          }
          const uint64_t m = __ballot(lane < (int)cnt && gt < krem && krem <= ge);
          const int src = m ? __builtin_ctzll(m) : 0;
          const uint32_t K = __shfl(mine, src, 64), g = __shfl(gt, src, 64);
          if (lane == 0) {
            lds.chosen[0] = K;
            lds.chosen[1] = g;
          }
        }
        __syncthreads();
        prefix = lds.chosen[0];
        pmask = ~0u;
        krem -= lds.chosen[1];
        __syncthreads();
        top = 0;
      }
    }
  };

  // Writes the selection from gathered lists (wavefront w's keys in
  // ckey[w*R, w*R + cand_cnt[w]), the lists together in column order): the
  // keys above K and the first keq (by column) equal to it.
  auto write_list = [&](const uint32_t* ckey, const int32_t* ccol, uint32_t R, uint32_t K,
                        uint32_t keq) {
    const uint32_t cnt = lds.cand_cnt[wave];
    uint32_t g = 0, q = 0;
    for (uint32_t c = lane; c < cnt; c += 64) {
      const uint32_t key = ckey[wave * R + c];
      g += key > K ? 1u : 0u;
      q += key == K ? 1u : 0u;
    }
    g = wave_sum(g);
    q = wave_sum(q);
    if (lane == 0) {
      lds.wave_gt[wave] = g;
      lds.wave_eq[wave] = q;
    }
    __syncthreads();
    uint32_t pos = 0, eq_rank = 0;
    for (int w = 0; w < wave; ++w) {
      const uint32_t gw = lds.wave_gt[w], qw = lds.wave_eq[w];
      pos += gw + (eq_rank < keq ? min(qw, keq - eq_rank) : 0u);
      eq_rank += qw;
    }
    for (uint32_t c0l = 0; c0l < cnt; c0l += 64) {
      const uint32_t c = c0l + lane;
      const bool in = c < cnt;
      const uint32_t key = in ? ckey[wave * R + c] : 0u;
      const uint64_t be = __ballot(in && key == K);
      const uint32_t my_eq = eq_rank + lanes_below(be);
      const bool sel = in && (key > K || (key == K && my_eq < keq));
      const uint64_t bs = __ballot(sel);
      const uint32_t p = pos + lanes_below(bs);
      if (sel && p < (uint32_t)k) {
        oi[p] = ccol[wave * R + c];
        if (ov) ov[p] = __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
      }
      pos += __builtin_popcountll(bs);
      eq_rank += __builtin_popcountll(be);
    }
  };

  // A split row whose lists are whole: the plan kernel set a threshold no
  // larger than the k-th largest key (checked here: at least k keys reach
  // it), and the gather kernel listed every key at or above it, chunk by
  // chunk in column order.  The selection is made on the list alone.
  const uint32_t thr = ws.map && !staged ? ws.thr[r] : kNoSplit;
  if (thr != kNoSplit) {
    const int32_t C = chunk_cols(n), nch = (n + C - 1) / C;
    if (tid < nch) {
      const int32_t m = ws.cnt[r * kMaxChunks + tid];
      const int32_t lo = chunk_slot(tid * C, tid, n);
      const int32_t size = chunk_slot(min(n, (tid + 1) * C), tid + 1, n) - lo;
      lds.chunk_lo[tid] = lo;
      lds.chunk_cnt[tid] = (m >= 0 && m <= size) ? m : -1;  // -1: the list overflowed
    }
    __syncthreads();
    int32_t total = 0;
    bool whole = true;
    for (int j = 0; j < nch; ++j) {
      const int32_t m = lds.chunk_cnt[j];
      whole = whole && m >= 0;
      total += max(m, 0);
    }
    if (whole && total >= k && total <= long_cap<kSelThreads>()) {
      uint32_t* ckey = lds.cand_long.key;
      int32_t* ccol = lds.cand_long.col;
      const uint32_t R = (uint32_t)long_cap<kSelThreads>() / kSelWaves;
      // entry i of the joined list goes to slot i: wavefront i / R's list
      // (the reads of a round are all issued before the LDS writes)
      constexpr int kU = (long_cap<kSelThreads>() + kSelThreads - 1) / kSelThreads;
      uint32_t kk[kU];
      int32_t cc[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t i = tid + u * kSelThreads;
        if (i < total) {
          int32_t j = 0, before = 0;
          while (before + lds.chunk_cnt[j] <= i) before += lds.chunk_cnt[j++];
          const int64_t g = r * kRowSlots + lds.chunk_lo[j] + (i - before);
          kk[u] = ws.key[g];
          cc[u] = ws.col[g];
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t i = tid + u * kSelThreads;
        if (i < total) {
          ckey[i] = kk[u];
          ccol[i] = cc[u];
        }
      }
      // the bits above the highest one where some listed key differs from
      // the threshold are the threshold's (the keys of a row's top few
      // percent share their sign and most exponent bits, which would put
      // them all in a few bins of a first digit taken from the top)
      uint32_t diff = 0;
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (tid + u * kSelThreads < total) diff |= kk[u] ^ thr;
      for (int off = 1; off < 64; off <<= 1) diff |= __shfl_xor(diff, off, 64);
      if (lane == 0) lds.wave_sum[wave] = diff;
      if (lane == 0)
        lds.cand_cnt[wave] = (uint32_t)min(max(total - wave * (int32_t)R, 0), (int32_t)R);
      __syncthreads();
      diff = 0;
      for (int w = 0; w < kSelWaves; ++w) diff |= lds.wave_sum[w];
      const int top = diff ? 32 - __builtin_clz(diff) : 0;
      uint32_t pmask = top == 32 ? 0u : ~0u << top, prefix = thr & pmask, krem = (uint32_t)k;
      __syncthreads();  // wave_sum is read before choose_bin writes it
      resolve(ckey, R, top, pmask, prefix, krem, kTopBits, lds.hist, (uint32_t)total);
      write_list(ckey, ccol, R, prefix, krem);
      return;
    }
    __syncthreads();  // the counts above are read before the path below reuses LDS
  }

  if (fast_list<kSelThreads>(fast, row, n, k, oi, ov)) return;

  // 0. A row not kept in LDS is sampled first (256 contiguous columns of
  //    every 4096, so every read is a whole 1 KB line run): the first-digit
  //    bins that hold the k-th largest key with high probability (its rank
  //    in the sample +- 4 standard deviations, at most kWin bins) get a
  //    histogram of the second digit during pass 1.  A sample that misses
  //    only costs the faster path below.
  uint32_t wlo = 1, whi = 0;  // the window [wlo, whi], empty
  uint32_t* fine = reinterpret_cast<uint32_t*>(lds.stage);  // [kWin][kBins2]
  for (int j = tid; j < kBins; j += kSelThreads) lds.hist[j] = 0;
  if (!staged)
    for (int j = tid; j < kWin * kBins2; j += kSelThreads) fine[j] = 0;
  if (tid == 0) lds.chosen[0] = lds.chosen[1] = lds.chosen[2] = 0;
  __syncthreads();
  if (!staged) {
    for_each_sample<kSelThreads, kSampleRun>(row, lds, n, [&](int32_t col, const v4f& v) {
      uint32_t bin[4];
      bool act[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bin[e] = order_key(v[e]) >> kTopShift;
        act[e] = col + e < n;
      }
      hist_add4(lds.hist, bin, act);
    });
    __syncthreads();
    const int32_t ns = sample_size<kSampleRun>(n);
    const float ks = (float)k * (float)ns / (float)n;
    const float m = 4.f * sqrtf(ks) + 4.f;
    const uint32_t r_hi = (uint32_t)max(1.f, floorf(ks - m));
    const uint32_t r_lo = (uint32_t)min((float)ns, ceilf(ks + m));
    choose_bin<kSelThreads>(lds, lds.hist, kBins, r_hi);
    whi = lds.chosen[0];
    __syncthreads();
    choose_bin<kSelThreads>(lds, lds.hist, kBins, r_lo);
    wlo = max(lds.chosen[0], whi >= kWin - 1 ? whi - (kWin - 1) : 0u);
    __syncthreads();
    for (int j = tid; j < kBins; j += kSelThreads) lds.hist[j] = 0;
    if (tid == 0) lds.chosen[0] = lds.chosen[1] = lds.chosen[2] = 0;
    __syncthreads();
  }

  // 1. Histogram of the top digit (and the LDS copy of a short row, or the
  //    second-digit histograms of the window).
  for_each_tile(row, lds, false, c0, c1, [&](int32_t i, const v4f& v) {
    if (staged && i < c1) {
      if (i + 4 <= c1) {
        *reinterpret_cast<v4f*>(lds.stage + i) = v;
      } else {
        for (int e = 0; e < 4; ++e)
          if (i + e < c1) lds.stage[i + e] = v[e];
      }
    }
    uint32_t bin[4], fbin[4];
    bool in[4], inw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = order_key(v[e]);
      bin[e] = key >> kTopShift;
      in[e] = i + e < c1;
      fbin[e] = (bin[e] - wlo) * kBins2 + ((key >> (kTopShift - 8)) & 0xFFu);
      inw[e] = in[e] & (bin[e] >= wlo) & (bin[e] <= whi);
    }
    hist_add4(lds.hist, bin, in);
    hist_add4(fine, fbin, inw);
  });
  __syncthreads();
  choose_bin<kSelThreads>(lds, lds.hist, kBins, (uint32_t)k);
  const uint32_t b1 = lds.chosen[0];
  uint32_t krem = (uint32_t)k - lds.chosen[1];
  const uint32_t h1 = lds.chosen[2];
  __syncthreads();

  // 1b. The window held the k-th largest key: its top 19 bits are known
  //     now, and one more pass gathers every key at or above them (at most
  //     k - 1 above plus the few sharing them) in column order; the k-th key
  //     and the ordered write then work on that list alone.
  if (b1 >= wlo && b1 <= whi && h1 != krem) {
    choose_bin<kSelThreads>(lds, fine + (b1 - wlo) * kBins2, kBins2, krem);
    const uint32_t b2 = lds.chosen[0];
    uint32_t krem2 = krem - lds.chosen[1];
    const uint32_t h2 = lds.chosen[2];
    __syncthreads();  // the gather below overwrites the window histograms
    constexpr int kShift2 = kTopShift - 8;
    uint32_t pmask2 = ~0u << kShift2, prefix2 = ((b1 << 8) | b2) << kShift2;
    const uint32_t R = (uint32_t)long_cap<kSelThreads>() / kSelWaves;
    uint32_t* ckey = lds.cand_long.key;
    int32_t* ccol = lds.cand_long.col;
    // the histograms give the number of keys at or above prefix2 (k - krem2
    // above it, h2 sharing it): a list that cannot hold them is not gathered
    if ((uint32_t)k - krem2 + h2 <= R * kSelWaves) {  // uniform
      uint32_t mine = 0;
      for_each_tile(row, lds, false, c0, c1, [&](int32_t i, const v4f& v) {
        uint64_t bc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bc[e] = __ballot(i + e < c1 && order_key(v[e]) >= prefix2);
        uint32_t slot = mine;
#pragma unroll
        for (int e = 0; e < 4; ++e) slot += lanes_below(bc[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (((bc[e] >> lane) & 1u) && slot < R) {
            ckey[wave * R + slot] = order_key(v[e]);
            ccol[wave * R + slot] = i + e;
          }
          slot += (bc[e] >> lane) & 1u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) mine += __builtin_popcountll(bc[e]);
      });
      if (lane == 0) lds.cand_cnt[wave] = mine;
      __syncthreads();
      bool overflow = false;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) overflow = overflow || lds.cand_cnt[w] > R;
      if (!overflow) {
        resolve(ckey, R, kShift2, pmask2, prefix2, krem2);
        // prefix2 is the k-th largest key K; krem2 keys equal to it are taken
        write_list(ckey, ccol, R, prefix2, krem2);
        return;
      }
      __syncthreads();  // the list is abandoned; the path below reuses its space
    }
  }

  // 2. The k-th largest key K (bits under pmask, the others free) and the
  //    per-wavefront counts of keys above K and equal to K.
  uint32_t pmask = ~0u << kTopShift, prefix = b1 << kTopShift;
  bool counted = false;
  // Wavefront w appends the keys of bin b1 it finds to its own region of
  // the candidate buffer (R entries), so the gather needs no atomics; a
  // region that would overflow sends the row down the slower path.
  uint32_t* ckey = staged ? lds.cand.key : lds.cand_long.key;
  int32_t* ccol = staged ? lds.cand.col : lds.cand_long.col;
  const uint32_t R = (staged ? (uint32_t)kCand : (uint32_t)long_cap<kSelThreads>()) / kSelWaves;
  if (h1 != krem && h1 <= R * kSelWaves) {
    // gather bin b1; count the keys above it per wavefront
    uint32_t above = 0, mine = 0;  // mine: this wavefront's candidates so far
    for_each_tile(row, lds, staged, c0, c1, [&](int32_t i, const v4f& v) {
      uint64_t bc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t bin = order_key(v[e]) >> kTopShift;
        const bool in = i + e < c1;
        above += (in && bin > b1) ? 1u : 0u;
        bc[e] = __ballot(in && bin == b1);
      }
      uint32_t slot = mine;
#pragma unroll
      for (int e = 0; e < 4; ++e) slot += lanes_below(bc[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (((bc[e] >> lane) & 1u) && slot < R) {
          ckey[wave * R + slot] = order_key(v[e]);
          ccol[wave * R + slot] = i + e;
        }
        slot += (bc[e] >> lane) & 1u;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) mine += __builtin_popcountll(bc[e]);
    });
    above = wave_sum(above);
    if (lane == 0) {
      lds.wave_gt[wave] = above;
      lds.cand_cnt[wave] = mine;
    }
    __syncthreads();
    bool overflow = false;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) overflow = overflow || lds.cand_cnt[w] > R;
    if (!overflow) {
      // resolve the low 21 bits on the gathered keys: digits of 8, 8, 5 bits
      resolve(ckey, R, kTopShift, pmask, prefix, krem);
      // each wavefront counts its own candidates above K and equal to K
      uint32_t g = 0, q = 0;
      for (uint32_t c = lane; c < lds.cand_cnt[wave]; c += 64) {
        const uint32_t key = ckey[wave * R + c];
        g += key > prefix ? 1u : 0u;
        q += key == prefix ? 1u : 0u;
      }
      g = wave_sum(g);
      q = wave_sum(q);
      if (lane == 0) {
        lds.wave_gt[wave] += g;
        lds.wave_eq[wave] = q;
      }
      __syncthreads();
      counted = true;
    }
  }
  if (!counted && h1 != krem) {
    // a crowded bin: the other 21 bits in two more passes over the row,
    // digits of 11 and 10 bits counted in the first digit's histogram space
    // (free now: the chosen bin is read, a staged row's gather is over)
    static_assert(kTopShift <= 2 * kTopBits, "two digits of at most kTopBits bits");
    for (int top = kTopShift; top > 0;) {
      const int shift = max(top - kTopBits, 0);
      const uint32_t dmask = (1u << (top - shift)) - 1u;
      for (int j = tid; j <= (int)dmask; j += kSelThreads) lds.hist[j] = 0;
      __syncthreads();
      for_each_tile(row, lds, staged, c0, c1, [&](int32_t i, const v4f& v) {
        uint32_t bin[4];
        bool act[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = order_key(v[e]);
          bin[e] = (key >> shift) & dmask;
          act[e] = (i + e < c1) & ((key & pmask) == prefix);
        }
        hist_add4(lds.hist, bin, act);
      });
      __syncthreads();
      choose_bin<kSelThreads>(lds, lds.hist, (int)dmask + 1, krem);
      prefix |= lds.chosen[0] << shift;
      pmask |= dmask << shift;
      const uint32_t h = lds.chosen[2];
      krem -= lds.chosen[1];
      __syncthreads();
      if (h == krem) break;  // the chosen bin is taken whole
      top = shift;
    }
  }
  // Selected: keys whose bits under pmask exceed prefix, and the first krem
  // (in column order) of those equal to it.
  const uint32_t need_eq = krem;
  if (!counted) {
    uint32_t gt = 0, eq = 0;
    for_each_tile(row, lds, staged, c0, c1, [&](int32_t i, const v4f& v) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = order_key(v[e]) & pmask;
        const bool in = i + e < c1;
        gt += (in && key > prefix) ? 1u : 0u;
        eq += (in && key == prefix) ? 1u : 0u;
      }
    });
    gt = wave_sum(gt);
    eq = wave_sum(eq);
    if (lane == 0) {
      lds.wave_gt[wave] = gt;
      lds.wave_eq[wave] = eq;
    }
    __syncthreads();
  }

  // 3. Ordered write.  Output position and equal-key rank at the start of
  //    this wavefront's chunk:
  uint32_t pos = 0, eq_rank = 0;
  for (int w = 0; w < wave; ++w) {
    const uint32_t g = lds.wave_gt[w], q = lds.wave_eq[w];
    pos += g + (eq_rank < need_eq ? min(q, need_eq - eq_rank) : 0u);
    eq_rank += q;
  }
  for_each_tile(row, lds, staged, c0, c1, [&](int32_t i, const v4f& v) {
    if (pos >= (uint32_t)k) return;  // uniform: the wavefront's share is written
    uint64_t bg[4], be[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = order_key(v[e]) & pmask;
      const bool in = i + e < c1;
      bg[e] = __ballot(in && key > prefix);
      be[e] = __ballot(in && key == prefix);
    }
    // column i+e of lane l follows every column of the lanes below l and
    // columns i..i+e-1 of lane l
    uint32_t eq_before = 0, eq_total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      eq_before += lanes_below(be[e]);
      eq_total += __builtin_popcountll(be[e]);
    }
    uint32_t my_eq = eq_rank + eq_before;
    uint32_t sel = 0;  // bit e: column i+e selected
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool g = (bg[e] >> lane) & 1u, q = (be[e] >> lane) & 1u;
      if (g || (q && my_eq < need_eq)) sel |= 1u << e;
      my_eq += q ? 1u : 0u;
    }
    uint64_t bs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) bs[e] = __ballot((sel >> e) & 1u);
    uint32_t p = pos, total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p += lanes_below(bs[e]);
      total += __builtin_popcountll(bs[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (((sel >> e) & 1u) && p < (uint32_t)k) {
        oi[p] = i + e;
        if (ov) ov[p] = v[e];
        ++p;
      }
    }
    pos += total;
    eq_rank += eq_total;
  });

}

// Workgroups [0, groups) are groups: wavefront w of group g selects row
// g kSelWaves + w, unless the row has more than wave_cols candidates
// (kWaveCols at most).  Workgroup groups + r then selects row r, the whole
// workgroup on it, if it has more than wave_cols candidates, and exits at
// once otherwise; the
// dispatcher refills the freed slots with the next workgroups, so the wide
// rows start within a few microseconds.  With a split workspace the grid is
// one workgroup per row instead, in the order the plan kernel set.
template <int kSelThreads>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(8)))
void select_topk_kernel(const float* __restrict__ logits, int64_t ldo, int32_t rows,
                        int32_t groups, int32_t wave_cols, int32_t max_ctx,
                        const int32_t* __restrict__ lengths,
                        const int32_t* __restrict__ ctx, const int32_t* __restrict__ sched,
                        int32_t batch, int32_t next_n, int32_t workers, int32_t k,
                        int32_t* __restrict__ out_idx, float* __restrict__ out_val, int64_t ldk,
                        SplitWs ws) {
  constexpr int W = kSelThreads / 64;
  __shared__ union {
    SelLds<kSelThreads> sel;
    FastLds<kSelThreads> fast;
    WaveLds wv[W];
  } smem;
  // 160 KB of LDS per compute unit: four workgroups of 512 threads or two
  // of 1024 (eight wavefronts per SIMD)
  static_assert(sizeof(smem) <= 160 * 1024 * kSelThreads / 2048, "LDS of a workgroup");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto cands = [&](int64_t q) {
    return row_candidates((int32_t)q, max_ctx, lengths, ctx, sched, batch, next_n, workers);
  };
  if (ws.map) {
    // the split path: the plan kernel has ordered the rows and counted
    // their candidates
    const int64_t r = ws.map[blockIdx.x];
    select_row_wg<kSelThreads>(smem.sel, smem.fast, logits + r * ldo, r, ws.len[r], k,
                               out_idx + r * ldk, out_val ? out_val + r * ldk : nullptr, ws);
    return;
  }
  const int32_t g = (int32_t)blockIdx.x;
  if (g < groups) {
    const int64_t r = (int64_t)g * W + wave;
    if (r >= rows) return;
    const int32_t n = cands(r);
    if (n > wave_cols) return;  // a wide worker's
    if (n > 4096) __builtin_amdgcn_s_setprio(1);  // see the long rows' priority below
    select_row_wave(smem.wv[wave], logits + r * ldo, n, k, out_idx + r * ldk,
                    out_val ? out_val + r * ldk : nullptr);
    return;
  }
  const int64_t r = g - groups;
  const int32_t n = cands(r);
  if (n <= wave_cols) return;  // a group's
  // The rows that end last take the SIMDs' issue slots first: the
  // wavefronts of rows of more than 32768 candidates and of wavefront rows
  // of more than 4096 run at instruction priority 1 (the kernel is bound by
  // instruction issue; measured on MI355X, large_fp8: 29.1 -> 28.4 us per
  // call; priority 2 for the longest rows starves the wavefront rows and
  // costs 2-3 us).
  if (n > 32768) __builtin_amdgcn_s_setprio(1);
  select_row_wg<kSelThreads>(smem.sel, smem.fast, logits + r * ldo, r, n, k, out_idx + r * ldk,
                             out_val ? out_val + r * ldk : nullptr, SplitWs{});
}

// The split path's plan, before the gather and the selection:
//  * workgroup 0 orders the rows longest first (by count class: 0 for none,
//    else 1 + 4 floor(log2 n) + the two bits below the leading one; rows of
//    one class in any order) into ws.map, and lists
//    every chunk of every row not kept in LDS (ws.chunk, count in ws.hdr);
//  * workgroup 1 + r sets row r's candidate count and, for a row not kept
//    in LDS, the key threshold: from a sample of the row (256 of every 4096
//    columns), the top 19 bits of the sampled key of rank
//    ks + 4.5 sqrt(ks) + 4.5, ks = k * (sample size) / n, so that at least
//    k keys of the row reach it but for a 4.5-sigma miss, and about
//    (1 + 4.5 / sqrt(ks)) k (1.4 k for k = 2048) are expected to.  A row
//    whose expected list would not fit kListCap slots comfortably is not
//    split.
template <int kSelThreads>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(8)))
void select_plan_kernel(const float* __restrict__ logits, int64_t ldo, int32_t rows,
                        int32_t max_ctx, const int32_t* __restrict__ lengths,
                        const int32_t* __restrict__ ctx, const int32_t* __restrict__ sched,
                        int32_t batch, int32_t next_n, int32_t workers, int32_t k, SplitWs ws) {
  __shared__ SelLds<kSelThreads> lds;
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    uint8_t* cls = reinterpret_cast<uint8_t*>(lds.stage);  // class of each row
    if (tid < kOrderBins) lds.hist[tid] = 0;
    if (tid == 0) lds.chosen[2] = 0;
    __syncthreads();
    for (int32_t q = tid; q < rows; q += kSelThreads) {
      const int32_t n = row_candidates(q, max_ctx, lengths, ctx, sched, batch, next_n, workers);
      const uint32_t c = count_class(n);
      cls[q] = (uint8_t)c;
      atomicAdd(&lds.hist[c], 1u);
      if (n > k && n > kStage) {
        const int32_t C = chunk_cols(n), nch = (n + C - 1) / C;
        const uint32_t base = atomicAdd(&lds.chosen[2], (uint32_t)nch);
        for (int32_t j = 0; j < nch; ++j) ws.chunk[base + j] = (q << 4) | j;
      }
    }
    __syncthreads();
    if (tid == 0) ws.hdr[0] = (int32_t)lds.chosen[2];
    if (tid < 64) {  // first rank of each class, from the top class down
      const int lane = tid;
      const uint32_t h0 = lds.hist[kOrderBins - 1 - 2 * lane];
      const uint32_t h1 = lds.hist[kOrderBins - 2 - 2 * lane];
      const uint32_t own = h0 + h1;
      uint32_t incl = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      lds.hist2[kOrderBins - 1 - 2 * lane] = incl - own;
      lds.hist2[kOrderBins - 2 - 2 * lane] = incl - own + h0;
    }
    __syncthreads();
    for (int32_t q = tid; q < rows; q += kSelThreads)
      ws.map[atomicAdd(&lds.hist2[cls[q]], 1u)] = q;
    return;
  }
  const int32_t r = (int32_t)blockIdx.x - 1;
  const int32_t n = row_candidates(r, max_ctx, lengths, ctx, sched, batch, next_n, workers);
  uint32_t thr = kNoSplit;
  if (n > k && n > kStage) {
    const float* row = logits + (int64_t)r * ldo;
    for (int j = tid; j < kBins; j += kSelThreads) lds.hist[j] = 0;
    if (tid < kBins2) lds.hist2[tid] = 0;
    __syncthreads();
    for_each_sample<kSelThreads, kPlanRun>(row, lds, n, [&](int32_t col, const v4f& v) {
      uint32_t bin[4];
      bool act[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bin[e] = order_key(v[e]) >> kTopShift;
        act[e] = col + e < n;
      }
      hist_add4(lds.hist, bin, act);
    });
    __syncthreads();
    const int32_t ns = sample_size<kPlanRun>(n);
    const float ks = (float)k * (float)ns / (float)n;
    const float rank = ceilf(ks + 4.5f * sqrtf(ks) + 4.5f);
    if (rank < (float)ns && rank * (float)n <= kListFill * (float)kListCap * (float)ns) {
      const uint32_t want = (uint32_t)rank;
      choose_bin<kSelThreads>(lds, lds.hist, kBins, want);
      const uint32_t b = lds.chosen[0], above = lds.chosen[1];
      __syncthreads();
      for_each_sample<kSelThreads, kPlanRun>(row, lds, n, [&](int32_t col, const v4f& v) {
        uint32_t bin[4];
        bool act[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = order_key(v[e]);
          bin[e] = (key >> (kTopShift - 8)) & 0xFFu;
          act[e] = (col + e < n) & ((key >> kTopShift) == b);
        }
        hist_add4(lds.hist2, bin, act);
      });
      __syncthreads();
      choose_bin<kSelThreads>(lds, lds.hist2, kBins2, want - above);
      thr = (b << kTopShift) | (lds.chosen[0] << (kTopShift - 8));
    }
  }
  if (tid == 0) {
    ws.len[r] = n;
    ws.thr[r] = thr;
  }
}

// Wave-uniform read through the constant address space (a scalar load).
__device__ __forceinline__ int32_t sload(const int32_t* p) {
  return __builtin_amdgcn_readfirstlane(*(const __attribute__((address_space(4))) int32_t*)(p));
}

// The split path's gather: a persistent grid takes the plan's chunk list in
// turn; for chunk j of row r (columns [jC, min(n, (j+1)C))) of a split row,
// every key at or above the row's threshold goes, in column order, to the
// chunk's slots of the row's list, and the count of those keys to ws.cnt (a
// count above the chunk's slots marks the list as not whole).  Each
// workgroup requests its next chunk's threshold and length while it reads
// the current chunk.

template <int kSelThreads>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(8)))
void select_gather_kernel(const float* __restrict__ logits, int64_t ldo, SplitWs ws) {
  constexpr int kSelWaves = kSelThreads / 64;
  __shared__ SelLds<kSelThreads> lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t R = (uint32_t)kListCap / kSelWaves;  // LDS list of each wavefront
  uint32_t* ckey = lds.cand_long.key;
  int32_t* ccol = lds.cand_long.col;
  const int32_t total = sload(ws.hdr);
  const int32_t G = (int32_t)gridDim.x;
  int32_t c = (int32_t)blockIdx.x;
  if (c >= total) return;
  // the chunk in hand and the next one's list entry, one chunk ahead
  int32_t e = sload(ws.chunk + c);
  int32_t e_next = c + G < total ? sload(ws.chunk + c + G) : 0;
  const int32_t* thr_w = reinterpret_cast<const int32_t*>(ws.thr);
  uint32_t thr = (uint32_t)sload(thr_w + (e >> 4));
  int32_t n = sload(ws.len + (e >> 4));
  for (; c < total; c += G) {
    const int32_t r = e >> 4, j = e & 15;
    // request the next chunk's threshold and length, and the entry after it
    const bool more = c + G < total;
    const int32_t rn = e_next >> 4;
    const uint32_t thr_n = more ? (uint32_t)sload(thr_w + rn) : kNoSplit;
    const int32_t n_n = more ? sload(ws.len + rn) : 0;
    const int32_t e_nn = c + 2 * G < total ? sload(ws.chunk + c + 2 * G) : 0;
    if (thr != kNoSplit) {
      const int32_t C = chunk_cols(n);
      const int32_t s0 = j * C, s1 = min(n, s0 + C);
      const int32_t lo = chunk_slot(s0, j, n), size = chunk_slot(s1, j + 1, n) - lo;
      const int32_t L = ((s1 - s0 + kSelWaves - 1) / kSelWaves + 3) & ~3;
      const int32_t c0 = min(s1, s0 + wave * L), c1 = min(s1, c0 + L);
      const float* row = logits + (int64_t)r * ldo;
      uint32_t mine = 0;
      for_each_tile(row, lds, false, c0, c1, [&](int32_t i, const v4f& v) {
        uint64_t bc[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) bc[q] = __ballot(i + q < c1 && order_key(v[q]) >= thr);
        uint32_t slot = mine;
#pragma unroll
        for (int q = 0; q < 4; ++q) slot += lanes_below(bc[q]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (((bc[q] >> lane) & 1u) && slot < R) {
            ckey[wave * R + slot] = order_key(v[q]);
            ccol[wave * R + slot] = i + q;
          }
          slot += (bc[q] >> lane) & 1u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) mine += __builtin_popcountll(bc[q]);
      });
      if (lane == 0) lds.cand_cnt[wave] = mine;
      __syncthreads();
      uint32_t pos = 0, tot = 0;
      bool over = false;
      for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t m = lds.cand_cnt[w];
        pos += w < wave ? m : 0u;
        tot += m;
        over = over || m > R;
      }
      const uint32_t stored = min(mine, R);
      const int64_t base = (int64_t)r * kRowSlots + lo;
      for (uint32_t i = lane; i < stored; i += 64) {
        if (pos + i < (uint32_t)size) {
          ws.key[base + pos + i] = ckey[wave * R + i];
          ws.col[base + pos + i] = ccol[wave * R + i];
        }
      }
      if (tid == 0) ws.cnt[r * kMaxChunks + j] = over ? size + 1 : (int32_t)tot;
      __syncthreads();  // the next chunk reuses the LDS lists
    }
    e = e_next;
    thr = thr_n;
    n = n_n;
    e_next = e_nn;
  }
}

}  // namespace

namespace {

// Bytes of the split path's workspace for `rows` rows (any max_ctx and k).
constexpr int64_t split_ws_bytes(int64_t rows) {
  return 4 * (64 + 3 * ws_words(rows) + 2 * ws_words(rows * kMaxChunks) +
              2 * ws_words(rows * kRowSlots));
}

// Scratch of the allocation-free selection (select_topk_noalloc): the split
// workspace of the most rows that are ever split, ~24.6 MiB per device,
// held until the process ends.  Host code never passes this name to a
// kernel: it stands for the array only on the device; the address of each
// device's copy comes from hipGetSymbolAddress below.
constexpr int64_t kScratchBytes = split_ws_bytes(kSplitRows);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

size_t select_workspace_bytes(int32_t rows, int32_t max_ctx, int32_t k) {
  if (rows < 1 || rows > kSplitRows || max_ctx <= kSplitCols || max_ctx <= k) return 0;
  return (size_t)split_ws_bytes(rows);
}

size_t static_scratch_bytes() { return (size_t)kScratchBytes; }

hipError_t static_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
      // the address of this device's copy, looked up with the device current
      int cur = 0;
      hipError_t e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) hipSetDevice(cur);
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

// Workgroups of 1024 threads when every row can have one at once (two per
// compute unit), else of 512 (four per compute unit).  Measured on MI355X:
// 512 rows of up to 131072 columns (nearly all of them long) select in
// ~52-63 us with 1024 threads; 2048 rows of lognormal lengths up to 65536 in
// ~38 us with 512.  With a workspace, at most kSplitRows rows and rows that
// may be longer than kSplitCols (more than the listing path's 16-bit column
// offsets reach with 512 threads), the plan and gather kernels run first.
hipError_t launch_select_topk(const float* logits, int64_t ldo, int32_t rows, int32_t max_ctx,
                              const int32_t* lengths, const int32_t* ctx, const int32_t* sched,
                              int32_t batch, int32_t next_n, int32_t workers, int32_t k,
                              int32_t* out_idx, float* out_val, int64_t ldk, void* workspace,
                              int32_t cus, hipStream_t stream) {
  SplitWs ws = {};
  if (workspace && rows <= kSplitRows && max_ctx > kSplitCols && max_ctx > k) {
    ws = split_ws(workspace, rows);
    hipLaunchKernelGGL(select_plan_kernel<512>, dim3(rows + 1), dim3(512), 0, stream, logits,
                       ldo, rows, max_ctx, lengths, ctx, sched, batch, next_n, workers, k, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_gather_kernel<512>, dim3(4 * (cus > 0 ? cus : 1)), dim3(512), 0,
                       stream, logits, ldo, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t c = cus > 0 ? cus : 1;
  const bool big = (int64_t)rows <= 2 * c;  // 1024 threads: two workgroups per compute unit
  const int32_t waves = big ? 16 : 8;
  // When every row gets a workgroup at once, a row is done sooner by its
  // workgroup than by one wavefront: only rows that are copied whole (at
  // most k candidates) stay with the groups.  Measured on MI355X, k = 2048:
  // 64 rows of 6144 columns 24 -> 12 us, 64 rows of decode logits (lengths
  // up to 65536) 19 -> 13 us, 256 rows 24 -> 19 us; a single row of 3000
  // columns 8.5 -> 9.7 us.
  const int32_t wave_cols = big ? min(k, kWaveCols) : kWaveCols;
  // without a split workspace: groups of wavefronts, then one workgroup per
  // row for the wide rows
  const int32_t groups = ws.map ? 0 : (int32_t)(((int64_t)rows + waves - 1) / waves);
  const dim3 grid(ws.map ? rows : groups + rows);
  if (big)
    hipLaunchKernelGGL(select_topk_kernel<1024>, grid, dim3(1024), 0, stream, logits, ldo, rows,
                       groups, wave_cols, max_ctx, lengths, ctx, sched, batch, next_n, workers, k, out_idx,
                       out_val, ldk, ws);
  else
    hipLaunchKernelGGL(select_topk_kernel<512>, grid, dim3(512), 0, stream, logits, ldo, rows,
                       groups, wave_cols, max_ctx, lengths, ctx, sched, batch, next_n, workers, k, out_idx,
                       out_val, ldk, ws);
  return hipGetLastError();
}

}  // namespace pmqa
