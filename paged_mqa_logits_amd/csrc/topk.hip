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
// One workgroup of 512 or 1024 threads per row; wavefront w owns the
// contiguous chunk [w*L, (w+1)*L) of the row's columns in every pass, 4
// columns per lane per 16-byte read.  Values are mapped to order-preserving
// 32-bit keys.
//   1. One read of the row (copied into LDS when it has at most 7680
//      columns) builds a histogram of the keys' top 11 bits; the bin that
//      holds the k-th largest key is b.
//   2. A second pass gathers the keys of bin b with their columns (when
//      there are at most 1024 of them, or 3840 -- 7680 with 1024 threads --
//      for a row not copied to LDS, whose gather goes where the copy would
//      be) and counts, per wavefront,
//      the keys above bin b.  The remaining 21 bits of the k-th largest key
//      K are found on the gathered list alone, which also gives each
//      wavefront's count of keys above K and equal to K.  (A larger bin is
//      resolved with further digit passes over the row and a counting pass
//      instead.)
//   3. A last pass writes the selected columns in order: keys above K, and
//      the first ones (by column) equal to K; each wavefront starts at the
//      output position the counts give it and ranks its columns with
//      ballots.
// A row not copied to LDS is sampled before step 1 (256 of every 4096
// columns) to guess the bins near the k-th key; step 1 then also histograms
// the next 8 bits of those bins, so when the guess holds, the k-th key's top
// 19 bits are known after step 1, step 2 gathers every key at or above them
// (the k - 1 above plus the few sharing them) in column order, and steps 2-3
// run on that list without reading the row a third time.  A guess that
// misses, or a list that would overflow a wavefront's share, takes the path
// above.
// Every pass reads 8 tiles ahead (8 16-byte reads in flight per lane for a
// row in global memory; after the first pass they hit L2).
//
// Rows are taken longest first: a row's time grows with its candidate
// count, and the dispatcher starts workgroups in index order, so workgroup i
// selects for the row of rank i in decreasing candidate count (by a coarse
// class: the top 3 bits of the count; ties by row index).  The longest rows
// then start at once instead of whenever their index comes up.  Each
// workgroup derives its row from the counts of all rows (for up to 8192
// rows; beyond that workgroup i takes row i).
//
// Split rows.  With a workspace and few rows (at most 512, two per compute
// unit, so one workgroup per row would leave most of the chip waiting on the
// longest rows), two kernels run before the selection:
//   * the plan orders the rows once for all workgroups (ws.map) and gives
//     each row not kept in LDS a key threshold from a sample of the row,
//     chosen so that at least k keys reach it (but for a miss of several
//     standard deviations) and about 1.4 k are expected to;
//   * the gather reads every such row in chunks of 16384 columns or more
//     (a persistent grid takes the plan's list of chunks in turn, each
//     workgroup requesting its next chunk's threshold while it reads the
//     current one) and lists the keys at or above the threshold, in column
//     order, with their count per chunk.
// The selection then takes a split row's list (a few thousand keys) instead
// of the row, resolves the k-th key on it and writes from it.  A list that
// is not whole (a chunk with more keys than its slots) or holds fewer than k
// keys (the sample missed) sends the row down the path above; either way the
// result is the same.
#include <hip/hip_runtime.h>

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
constexpr int kMaxChunks = 16;           // chunks of a split row, at most
constexpr int32_t kChunkMin = 16384;     // columns of a chunk, at least
constexpr int kRowSlots = 3 * kListCap / 2 + 32 * kMaxChunks;  // list slots of a row
constexpr uint32_t kNoSplit = 0xFFFFFFFFu;  // threshold of a row that is not split
constexpr int kPlanRun = 256;            // the plan samples 256 of every 4096 columns
constexpr float kListFill = 0.8f;        // expected list at most this share of kListCap

typedef float v4f __attribute__((ext_vector_type(4)));

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

constexpr int kOrderRows = 8192;          // rows ordered longest first
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

int64_t ws_words(int64_t n) { return (n + 63) & ~(int64_t)63; }

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

// The row of rank `rank` in decreasing count class (ties: lower row first);
// rows <= kOrderRows.  Every thread calls it; LDS is free on return.
template <int kSelThreads, class Lds>
__device__ __forceinline__ int32_t row_of_rank(Lds& lds, int32_t rank, int32_t rows,
                                            int32_t max_ctx, const int32_t* lengths,
                                            const int32_t* ctx, const int32_t* sched,
                                            int32_t batch, int32_t next_n, int32_t workers) {
  constexpr int kSelWaves = kSelThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint8_t* cls = reinterpret_cast<uint8_t*>(lds.stage);  // class of each row
  uint32_t* hist = lds.hist;
  if (tid < kOrderBins) hist[tid] = 0;
  __syncthreads();
  for (int32_t q = tid; q < rows; q += kSelThreads) {
    const uint32_t c =
        count_class(row_candidates(q, max_ctx, lengths, ctx, sched, batch, next_n, workers));
    cls[q] = (uint8_t)c;
    atomicAdd(&hist[c], 1u);
  }
  __syncthreads();
  // class holding the rank, counted from the top class down, and the rank
  // of its first row
  if (wave == 0) {
    const uint32_t h0 = hist[kOrderBins - 1 - 2 * lane], h1 = hist[kOrderBins - 2 - 2 * lane];
    const uint32_t own = h0 + h1;
    uint32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const uint32_t above = incl - own, rk = (uint32_t)rank;
    if (above <= rk && rk < above + h0) {
      lds.chosen[0] = kOrderBins - 1 - 2 * lane;
      lds.chosen[1] = above;
    } else if (above + h0 <= rk && rk < incl) {
      lds.chosen[0] = kOrderBins - 2 - 2 * lane;
      lds.chosen[1] = above + h0;
    }
  }
  __syncthreads();
  const uint32_t want_cls = lds.chosen[0], j = (uint32_t)rank - lds.chosen[1];
  // the j-th row of that class in row order, 512 rows per round
  uint32_t base = 0;
  for (int32_t r0 = 0; r0 < rows; r0 += kSelThreads) {
    const int32_t q = r0 + tid;
    const bool in = q < rows && cls[q] == want_cls;
    const uint64_t m = __ballot(in);
    if (lane == 0) lds.wave_sum[wave] = __builtin_popcountll(m);
    __syncthreads();
    uint32_t before = base, total = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      before += w < wave ? lds.wave_sum[w] : 0u;
      total += lds.wave_sum[w];
    }
    if (in && before + lanes_below(m) == j) lds.chosen[2] = (uint32_t)q;
    base += total;
    __syncthreads();
    if (base > j) break;  // uniform
  }
  const int32_t r = (int32_t)lds.chosen[2];
  __syncthreads();
  return r;
}

template <int kSelThreads>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu(8)))
void select_topk_kernel(const float* __restrict__ logits, int64_t ldo, int32_t max_ctx,
                        const int32_t* __restrict__ lengths, const int32_t* __restrict__ ctx,
                        const int32_t* __restrict__ sched, int32_t batch, int32_t next_n,
                        int32_t workers, int32_t k, int32_t* __restrict__ out_idx,
                        float* __restrict__ out_val, int64_t ldk, SplitWs ws) {
  constexpr int kSelWaves = kSelThreads / 64;
  __shared__ SelLds<kSelThreads> lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t rows = (int32_t)gridDim.x;
  // with the split workspace, the plan kernel has ordered the rows and
  // counted their candidates
  const int64_t r = ws.map ? (int64_t)ws.map[blockIdx.x]
                    : rows <= kOrderRows
                        ? row_of_rank<kSelThreads>(lds, (int32_t)blockIdx.x, rows, max_ctx,
                                                   lengths, ctx, sched, batch, next_n, workers)
                        : (int64_t)blockIdx.x;
  const float* row = logits + r * ldo;
  int32_t* oi = out_idx + r * ldk;
  float* ov = out_val ? out_val + r * ldk : nullptr;
  const int32_t n = ws.map ? ws.len[r]
                           : row_candidates((int32_t)r, max_ctx, lengths, ctx, sched, batch,
                                            next_n, workers);
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
        if (c % R < lds.cand_cnt[c / R] && (key & pmask) == prefix)
          atomicAdd(&hist[(key >> shift) & dmask], 1u);
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
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < n) atomicAdd(&lds.hist[order_key(v[e]) >> kTopShift], 1u);
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
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i + e < c1) {
        const uint32_t key = order_key(v[e]);
        const uint32_t bin = key >> kTopShift;
        atomicAdd(&lds.hist[bin], 1u);
        if (bin >= wlo && bin <= whi)
          atomicAdd(&fine[(bin - wlo) * kBins2 + ((key >> (kTopShift - 8)) & 0xFFu)], 1u);
      }
    }
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
    __syncthreads();  // the gather below overwrites the window histograms
    constexpr int kShift2 = kTopShift - 8;
    uint32_t pmask2 = ~0u << kShift2, prefix2 = ((b1 << 8) | b2) << kShift2;
    const uint32_t R = (uint32_t)long_cap<kSelThreads>() / kSelWaves;
    uint32_t* ckey = lds.cand_long.key;
    int32_t* ccol = lds.cand_long.col;
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
    // a crowded bin: further digits (8, 8, 5 bits) with passes over the row
    for (int top = kTopShift; top > 0;) {
      const int shift = max(top - 8, 0);
      const uint32_t dmask = (1u << (top - shift)) - 1u;
      if (tid < kBins2) lds.hist2[tid] = 0;
      __syncthreads();
      for_each_tile(row, lds, staged, c0, c1, [&](int32_t i, const v4f& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = order_key(v[e]);
          if (i + e < c1 && (key & pmask) == prefix)
            atomicAdd(&lds.hist2[(key >> shift) & dmask], 1u);
        }
      });
      __syncthreads();
      choose_bin<kSelThreads>(lds, lds.hist2, (int)dmask + 1, krem);
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

// The split path's plan, before the gather and the selection:
//  * workgroup 0 orders the rows longest first (by count class, as
//    row_of_rank; rows of one class in any order) into ws.map, and lists
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
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (col + e < n) atomicAdd(&lds.hist[order_key(v[e]) >> kTopShift], 1u);
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
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = order_key(v[e]);
          if (col + e < n && (key >> kTopShift) == b)
            atomicAdd(&lds.hist2[(key >> (kTopShift - 8)) & 0xFFu], 1u);
        }
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

size_t select_workspace_bytes(int32_t rows, int32_t max_ctx, int32_t k) {
  if (rows < 1 || rows > kSplitRows || max_ctx <= kStage || max_ctx <= k) return 0;
  const int64_t words = 64 + 3 * ws_words(rows) + 2 * ws_words((int64_t)rows * kMaxChunks) +
                        2 * ws_words((int64_t)rows * kRowSlots);
  return (size_t)words * 4;
}

// Workgroups of 1024 threads when every row can have one at once (two per
// compute unit), else of 512 (four per compute unit): measured on MI355X,
// 512 rows of up to 131072 columns select in 90-110 us with 1024 threads
// against 104-130 us with 512, and 2048 rows of up to 65536 in 64 us with
// 512 against 84 us with 1024.
// With a workspace, at most kSplitRows rows (two per compute unit) and rows
// that may be too long for LDS, the plan and gather kernels run first; the
// gather runs four workgroups per compute unit.  With more rows every
// compute unit already holds several rows at once, and the single kernel is
// faster (measured on MI355X: 2048 rows of up to 65536 columns select in
// ~62 us alone against ~68 us split, 512 rows of up to 131072 in 92-113 us
// alone against 59-64 us split).
hipError_t launch_select_topk(const float* logits, int64_t ldo, int32_t rows, int32_t max_ctx,
                              const int32_t* lengths, const int32_t* ctx, const int32_t* sched,
                              int32_t batch, int32_t next_n, int32_t workers, int32_t k,
                              int32_t* out_idx, float* out_val, int64_t ldk, void* workspace,
                              int32_t cus, hipStream_t stream) {
  SplitWs ws = {};
  if (workspace && rows <= kSplitRows && max_ctx > kStage && max_ctx > k) {
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
  if ((int64_t)rows <= 2 * (int64_t)cus)
    hipLaunchKernelGGL(select_topk_kernel<1024>, dim3(rows), dim3(1024), 0, stream, logits, ldo,
                       max_ctx, lengths, ctx, sched, batch, next_n, workers, k, out_idx, out_val,
                       ldk, ws);
  else
    hipLaunchKernelGGL(select_topk_kernel<512>, dim3(rows), dim3(512), 0, stream, logits, ldo,
                       max_ctx, lengths, ctx, sched, batch, next_n, workers, k, out_idx, out_val,
                       ldk, ws);
  return hipGetLastError();
}

}  // namespace pmqa
