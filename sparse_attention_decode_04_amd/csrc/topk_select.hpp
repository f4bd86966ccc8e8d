// The top-k selection of one workgroup over a chunk of one row's candidates:
// its shared state, the counting select, the streamed selection from scores
// and the level body. Used by the top-k level kernel and by the kernel that
// runs a row's final level ahead of its attention.
// (The method is described at the top of topk.hip.)
#pragma once

#include "device_common.hpp"
#include "ds_rows_internal.hpp"
#include "select_common.hpp"

namespace ds {

constexpr int kBins = 1024;
constexpr uint32_t kFastBinMax = 256;   // largest bin the counting select ranks by comparisons
// A sampled threshold keeps the keys at or above the kSampleMin-th best of
// the 1024 samples (each thread's first key) at 32 keys per thread, about
// 2048 of 32768; with fewer keys per thread the target rises in proportion
// (sample_target), so that about 2048 are kept at any chunk size (at 8 per
// thread a fixed 64 kept about 512, under the 512 needed half of the time,
// and the selection then fell back to its slow path over every key).
constexpr uint32_t kSampleMin = 64;
template <int kPer>
__device__ __forceinline__ uint32_t sample_target(uint32_t nsamp) {
  static_assert(kPer >= 1 && kPer <= 32, "keys per thread");
  return min(nsamp, kSampleMin * (32u / kPer));
}
constexpr int kWaves = kTopkThreads / 64;
constexpr uint32_t kCompactPerWave = 512;                  // compaction capacity of one wave
constexpr int kCompactPerLane = kCompactPerWave / 64;      // 8 compacted keys per thread
constexpr uint32_t kSmallChunk = 4096;                     // chunks this small keep every key

// Block-wide scan of the 1024-bin histogram from the top bin down: thread t
// owns bin 1023 - t. Gives that bin's count h, the number of keys in higher
// bins (`above`), the largest count among bins >= it (`maxge`) and the total
// count. Contains one barrier; callers separate successive uses of wsum/wmax.
__device__ __forceinline__ void scan_bins(const uint32_t *hist, uint32_t *wsum, uint32_t *wmax, uint32_t tid,
                                          uint32_t &h, uint32_t &above, uint32_t &maxge, uint32_t &total) {
  const uint32_t lane = tid & 63, wave = tid >> 6;
  h = hist[kBins - 1 - tid];
  const uint32_t incl = wave_prefix_sum(h), imax = wave_prefix_max(h);
  if (lane == 63) { wsum[wave] = incl; wmax[wave] = imax; }
  __syncthreads();
  uint32_t pre = 0, premax = 0, all = 0;
#pragma unroll
  for (int v = 0; v < kWaves / 4; ++v) {
    const u32x4 s4 = reinterpret_cast<const u32x4 *>(wsum)[v];
    const u32x4 m4 = reinterpret_cast<const u32x4 *>(wmax)[v];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool before_me = static_cast<uint32_t>(4 * v + k) < wave;
      pre += before_me ? s4[k] : 0u;
      premax = before_me ? max(premax, m4[k]) : premax;
      all += s4[k];
    }
  }
  above = pre + incl - h;
  maxge = max(premax, imax);
  total = all;
}

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t sfx[kBins];
  uint32_t cursor[kBins];
  uint64_t cand[kTopkSortCap];
  union {
    uint64_t compact[kWaves * kCompactPerWave];               // wave regions of kept keys
    uint32_t ordl[kTopkThreads * kTopkPerThreadFirst];        // first-level fallback: all score bits
  };
  __attribute__((aligned(16))) uint32_t wsum[kWaves];
  __attribute__((aligned(16))) uint32_t wmax[kWaves];
  __attribute__((aligned(16))) uint32_t wcount[kWaves];
  uint64_t s_floor;                                          // candidate statistics of the level,
  uint32_t s_total, s_min1, s_max;                           // combined by LDS atomics
  uint64_t wkmin[kWaves], wkmax[kWaves];                     // radix fallback: key range per wave
  uint32_t count, lo, digit, above, bin, kept, maxbin, hist_total, viol;
};

// Suffix scan of the 1024-bin histogram by the first four waves, four bins
// per thread (thread t owns bins 1023 - 4t - k, k = 0..3, the top bin
// first), and the search for the bin d that holds the need-th key: writes
// sfx[b] (keys in bins above b) for every bin, digit = d, kept (keys in bins
// >= d), maxbin (largest count of a bin >= d) and hist_total. One barrier
// inside (the wave totals); the caller's next barrier publishes the results.
// Four waves with four bins each issue a fraction of the instructions that
// sixteen waves with one bin each (and a sixteen-way combine) would.
static_assert(kBins == 4 * 256 && kTopkThreads >= 256, "four waves, four bins per thread");
__device__ __forceinline__ void scan_digit(TopkShared &sh, uint32_t need, uint32_t tid) {
  const uint32_t lane = tid & 63, wave = tid >> 6;
  const bool mine = wave < 4;   // wave-uniform
  uint32_t v[4] = {0, 0, 0, 0}, sum = 0, m = 0, incl = 0, imax = 0;
  if (mine) {
    const u32x4 h4 = reinterpret_cast<const u32x4 *>(sh.hist)[255 - tid];   // bins 1020 - 4t .. 1023 - 4t
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = h4[3 - k];   // bin 1023 - 4t - k
      sum += v[k];
      m = max(m, v[k]);
    }
    incl = wave_prefix_sum(sum);
    imax = wave_prefix_max(m);
    if (lane == 63) { sh.wsum[wave] = incl; sh.wmax[wave] = imax; }
  }
  __syncthreads();
  if (mine) {
    const u32x4 s4 = reinterpret_cast<const u32x4 *>(sh.wsum)[0];
    const u32x4 m4 = reinterpret_cast<const u32x4 *>(sh.wmax)[0];
    uint32_t pre = 0, premax = 0, all = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool before_me = static_cast<uint32_t>(k) < wave;
      pre += before_me ? s4[k] : 0u;
      premax = before_me ? max(premax, m4[k]) : premax;
      all += s4[k];
    }
    // Largest count in the lanes before this one (their bins are all higher).
    const uint32_t prev_max = __shfl_up(imax, 1);
    uint32_t above = pre + incl - sum;   // keys in bins above this thread's first bin
    uint32_t maxge = max(premax, lane > 0 ? prev_max : 0u);
    u32x4 sfx4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t b = kBins - 1 - 4 * tid - k;
      maxge = max(maxge, v[k]);
      sfx4[3 - k] = above;
      if (above < need && need <= above + v[k]) {
        sh.digit = b;
        sh.kept = above + v[k];
        sh.maxbin = maxge;
      }
      above += v[k];
    }
    reinterpret_cast<u32x4 *>(sh.sfx)[255 - tid] = sfx4;
    if (tid == 0) sh.hist_total = all;
  }
}

// Candidates of the first level: score bits per candidate (0 = none), index
// implied by the position begin + tid + 1024 e.
template <int N>
struct OrdCand {
  uint32_t (&o)[N];
  uint32_t pos0;   // begin + tid
  __device__ __forceinline__ uint32_t hi(int e) const { return o[e]; }
  // ~position, rebuilt from one opaque base so that N positions are not kept
  // live from the loads on.
  __device__ __forceinline__ uint32_t low(int e) const {
    uint32_t nbase = ~pos0;
    asm volatile("" : "+v"(nbase));
    return nbase - kTopkThreads * static_cast<uint32_t>(e);
  }
  __device__ __forceinline__ uint64_t key(int e) const {
    return o[e] ? (static_cast<uint64_t>(o[e]) << 32) | low(e) : 0ull;
  }
  __device__ __forceinline__ uint64_t vkey(int e) const { return (static_cast<uint64_t>(o[e]) << 32) | low(e); }
  // Opaque register barrier: values derived from the keys (full keys, masks)
  // are recomputed after it rather than kept live across a loop.
  __device__ __forceinline__ void fence() const {
#pragma unroll
    for (int e = 0; e < N; ++e) asm volatile("" : "+v"(o[e]));
  }
};

// The same candidates after they were moved to LDS (ordl[tid + 1024 e]).
struct LdsOrdCand {
  const uint32_t *ordl;
  uint32_t tid, pos0;
  __device__ __forceinline__ uint32_t hi(int e) const { return ordl[tid + kTopkThreads * e]; }
  __device__ __forceinline__ uint32_t low(int e) const { return ~pos0 - kTopkThreads * static_cast<uint32_t>(e); }
  __device__ __forceinline__ uint64_t key(int e) const {
    const uint32_t o = hi(e);
    return o ? (static_cast<uint64_t>(o) << 32) | low(e) : 0ull;
  }
  __device__ __forceinline__ uint64_t vkey(int e) const { return (static_cast<uint64_t>(hi(e)) << 32) | low(e); }
  __device__ __forceinline__ void fence() const {}
};

// Candidates held as full 64-bit keys (0 = none).
template <int N>
struct KeyCand {
  uint64_t (&k)[N];
  __device__ __forceinline__ uint32_t hi(int e) const { return static_cast<uint32_t>(k[e] >> 32); }
  __device__ __forceinline__ uint64_t key(int e) const { return k[e]; }
  __device__ __forceinline__ uint64_t vkey(int e) const { return k[e]; }
  __device__ __forceinline__ void fence() const {
#pragma unroll
    for (int e = 0; e < N; ++e) asm volatile("" : "+v"(k[e]));
  }
};

// Best `need` of the workgroup's candidates (kPer per thread, read through
// `c`; their score bits lie in [omin, omax]), emitted in rank order through
// emit(pos, key). kSample: pre-filter the histogram by a sampled lower bin
// (worth it only for many candidates per thread).
// kFresh: hist, cursor, count and lo still hold the zeros written at the
// start of the kernel (published by a barrier since), and no earlier reader
// of the shared arrays remains, so they are not cleared again.
// kIntBins: bins of equal width in the score bits rather than in the score,
// (o - omin) >> shift: half the instructions per key and no division. Any
// binning that preserves the score order gives the same selection; this one
// suits candidates that are a row's best keys (a narrow range of scores),
// not raw scores around zero, whose bits span many binades.
template <int kPer, bool kSample, bool kFresh = false, bool kIntBins = false, class Cand, class Emit>
__device__ __forceinline__ void counting_select(TopkShared &sh, const Cand &c, uint32_t total, uint32_t need,
                                                uint32_t omin, uint32_t omax, const Emit &emit) {
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  if constexpr (!kFresh) {
    __syncthreads();   // earlier readers of the shared arrays are done
    sh.hist[tid] = 0;
    sh.cursor[tid] = 0;
    if (tid == 0) { sh.count = 0; sh.lo = 0; }
    __syncthreads();
  }

  static_assert(kBins == 1 << 10, "integer bins take the top 10 bits of the span");
  float smin = 0.0f, scale = 0.0f;
  uint32_t shift = 0;
  if constexpr (kIntBins) {
    // (omax - omin) >> shift < kBins; every valid key's bits lie in [omin, omax].
    const uint32_t span = omax - omin;
    shift = span < static_cast<uint32_t>(kBins) ? 0u : static_cast<uint32_t>(32 - __builtin_clz(span) - 10);
  } else {
    smin = ord_score(omin);
    const float range = ord_score(omax) - smin;
    scale = (range > 0.0f && __builtin_isfinite(range)) ? static_cast<float>(kBins) / range : 0.0f;
  }
  // Bin of a key's score bits o (nonzero: a valid key). A zero range gives
  // every (finite) key bin 0.
  auto bin_of = [&](uint32_t o) -> uint32_t {
    if constexpr (kIntBins) return (o - omin) >> shift;
    else return static_cast<uint32_t>(fminf((ord_score(o) - smin) * scale, static_cast<float>(kBins - 1)));
  };
  // Bin of every candidate, once, two 16-bit bins per register; kBins = no
  // key.
  uint32_t binp[kPer / 2];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const uint32_t o = c.hi(e);
    const uint32_t b = o != 0 ? bin_of(o) : static_cast<uint32_t>(kBins);
    if (e & 1) binp[e / 2] |= b << 16;
    else binp[e / 2] = b;
  }
  auto bin_at = [&](int e) -> uint32_t { return (e & 1) ? binp[e / 2] >> 16 : binp[e / 2] & 0xFFFFu; };
  // A bin b lies in [lo, kBins) iff b - lo < kBins - lo (unsigned).
  auto in_range = [](uint32_t b, uint32_t lo) { return b - lo < static_cast<uint32_t>(kBins) - lo; };

  uint32_t lo = 0;
  if constexpr (kSample) {
    // Sample (each thread's first key) -> likely lower bin lo.
    hist_add(sh.hist, bin_at(0), kBins, lane);
    __syncthreads();
    {
      uint32_t h, above, maxge, nsamp;
      scan_bins(sh.hist, sh.wsum, sh.wmax, tid, h, above, maxge, nsamp);
      const uint32_t target = sample_target<kPer>(nsamp);
      if (target > 0 && above < target && target <= above + h) sh.lo = kBins - 1 - tid;
    }
    __syncthreads();
    lo = sh.lo;
    sh.hist[tid] = 0;
    __syncthreads();
  }

  // Histogram of the keys in bins >= lo, scan; if they are fewer than need,
  // once more over every key (lo = 0).
  uint32_t d = 0, kept = 0, maxbin = 0;
  for (;;) {
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (in_range(bin_at(e), lo)) hist_add(sh.hist, bin_at(e), kBins, lane);
    __syncthreads();
    scan_digit(sh, need, tid);
    __syncthreads();
    if (sh.hist_total >= need || lo == 0) {
      d = sh.digit;
      kept = sh.kept;
      maxbin = sh.maxbin;
      break;
    }
    lo = 0;
    sh.hist[tid] = 0;
    __syncthreads();
  }
  if (kept <= kTopkSortCap && maxbin <= kFastBinMax) {
    // Scatter the keys of bins >= d grouped by bin, then rank within bins.
    c.fence();
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (in_range(bin_at(e), d)) sh.cand[sh.sfx[bin_at(e)] + atomicAdd(&sh.cursor[bin_at(e)], 1u)] = c.vkey(e);
    __syncthreads();
    if (tid < kept) {
      const uint64_t kk = sh.cand[tid];
      const uint32_t b = bin_of(static_cast<uint32_t>(kk >> 32));
      const uint32_t base = sh.sfx[b], n = sh.hist[b];
      uint32_t rank = 0;
      for (uint32_t q = 0; q < n; ++q) rank += sh.cand[base + q] > kk ? 1u : 0u;
      const uint32_t pos = base + rank;
      if (pos < need) emit(pos, kk);
    }
    return;
  }

  // ---- fallback: radix select on the 64-bit keys, then bitonic sort ------
  uint64_t thr = 1;
  if (total > kTopkSortCap) {
    // The passes start at the highest byte in which the smallest and the
    // largest candidate differ: heavy ties (equal scores) share their upper
    // bytes, which a pass would only confirm.
    uint64_t kmin = ~0ull, kmax = 0;
    c.fence();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint64_t kk = c.key(e);
      if (kk != 0) { kmin = min(kmin, kk); kmax = max(kmax, kk); }
    }
    {
      const uint32_t hmin = wave_min(static_cast<uint32_t>(kmin >> 32));
      const uint32_t lmin = wave_min(static_cast<uint32_t>(kmin >> 32) == hmin ? static_cast<uint32_t>(kmin) : ~0u);
      const uint32_t hmax = wave_max(static_cast<uint32_t>(kmax >> 32));
      const uint32_t lmax = wave_max(static_cast<uint32_t>(kmax >> 32) == hmax ? static_cast<uint32_t>(kmax) : 0u);
      if (lane == 0) {
        sh.wkmin[tid >> 6] = (static_cast<uint64_t>(hmin) << 32) | lmin;
        sh.wkmax[tid >> 6] = (static_cast<uint64_t>(hmax) << 32) | lmax;
      }
    }
    __syncthreads();
    kmin = ~0ull;
    kmax = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      kmin = min(kmin, sh.wkmin[w]);
      kmax = max(kmax, sh.wkmax[w]);
    }
    const uint64_t diff = kmin ^ kmax;   // nonzero: more than kTopkSortCap distinct keys
    const int top = diff == 0 ? 0 : (63 - __builtin_clzll(diff)) / 8 * 8;
    uint32_t left = kTopK;          // ranks still to fill below the prefix
    uint64_t prefix = top == 56 ? 0ull : (kmax >> (top + 8)) << (top + 8);   // the common upper bytes
    for (int shift = top; shift >= 0; shift -= 8) {
      __syncthreads();
      if (tid < 256) sh.hist[tid] = 0;
      __syncthreads();
      c.fence();
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const uint64_t kk = c.key(e);
        const bool match = kk != 0 && (shift == 56 || (kk >> (shift + 8)) == (prefix >> (shift + 8)));
        hist_add(sh.hist, match ? static_cast<uint32_t>(kk >> shift) & 255u : 256u, 256, lane);
      }
      __syncthreads();
      uint32_t t = tid;
      asm volatile("" : "+v"(t));   // keeps the digit arithmetic out of the loop preheader
      if (t < 64) {
        uint32_t v[4], sum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) { v[k] = sh.hist[255 - 4 * t - k]; sum += v[k]; }
        const uint32_t incl = wave_prefix_sum(sum);   // wave 0, every lane active
        uint32_t before = incl - sum;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (before < left && left <= before + v[k]) {
            sh.digit = 255 - 4 * t - k;
            sh.above = before;
            sh.bin = v[k];
          }
          before += v[k];
        }
      }
      __syncthreads();
      left -= sh.above;
      prefix |= static_cast<uint64_t>(sh.digit) << shift;
      if ((kTopK - left) + sh.bin <= kTopkSortCap) { thr = prefix; break; }
    }
  }
  c.fence();
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const uint64_t kk = c.key(e);
    if (kk != 0 && kk >= thr) {
      const uint32_t pos = atomicAdd(&sh.count, 1u);
      if (pos < kTopkSortCap) sh.cand[pos] = kk;   // at most 1024 by construction
    }
  }
  __syncthreads();
  const uint32_t nk = min(sh.count, static_cast<uint32_t>(kTopkSortCap));
  if (tid >= nk) sh.cand[tid] = 0;
  __syncthreads();
  const uint32_t size = nk <= kTopK ? kTopK : kTopkSortCap;
  for (uint32_t k = 2; k <= size; k <<= 1) {
    for (uint32_t j = k >> 1; j > 0; j >>= 1) {
      const uint32_t ixj = tid ^ j;
      if (tid < size && ixj > tid) {
        const uint64_t x = sh.cand[tid], y = sh.cand[ixj];
        const bool desc = (tid & k) == 0;
        if (desc ? (x < y) : (x > y)) { sh.cand[tid] = y; sh.cand[ixj] = x; }
      }
      __syncthreads();
    }
  }
  if (tid < need) emit(tid, sh.cand[tid]);
}

// Exact top-min(512, n) of n scores, streamed from memory by one workgroup:
// MSB-first 8-bit radix select on the 64-bit keys until at most 1024 keys lie
// at or above the prefix, then a bitonic sort of those in LDS. Used when the
// fused indexer's candidates cannot be shown to contain a row's top 512
// (heavy ties, sorted scores); slow but independent of the score
// distribution. Emits every slot (0 past the selected count).
template <class Emit>
__device__ __forceinline__ void select_from_scores(TopkShared &sh, const float *sc, uint32_t n, const Emit &emit) {
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  constexpr int kU = 8;   // loads in flight per thread
  const uint32_t last = n > 0 ? n - 1 : 0;
  auto keys = [&](uint32_t p0, uint64_t (&kk)[kU]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t p = p0 + u * kTopkThreads + tid;
      kk[u] = topk_key(sc[min(p, last)], p);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (p0 + u * kTopkThreads + tid >= n) kk[u] = 0;
  };
  uint64_t prefix = 0, thr = 1;
  uint32_t left = kTopK, total = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    __syncthreads();
    if (tid < 256) sh.hist[tid] = 0;
    if (tid == 0) sh.count = 0;
    __syncthreads();
    uint32_t nv = 0;
    for (uint32_t p0 = 0; p0 < n; p0 += kU * kTopkThreads) {
      uint64_t kk[kU];
      keys(p0, kk);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        nv += kk[u] != 0 ? 1u : 0u;
        const bool match = kk[u] != 0 && (shift == 56 || (kk[u] >> (shift + 8)) == (prefix >> (shift + 8)));
        hist_add(sh.hist, match ? static_cast<uint32_t>(kk[u] >> shift) & 255u : 256u, 256, lane);
      }
    }
    nv = wave_sum(nv);
    if (lane == 0) atomicAdd(&sh.count, nv);
    __syncthreads();
    total = sh.count;
    if (total <= kTopkSortCap) { thr = 1; break; }   // (the same on every pass)
    uint32_t t = tid;
    asm volatile("" : "+v"(t));
    if (t < 64) {
      uint32_t v[4], sum = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) { v[k] = sh.hist[255 - 4 * t - k]; sum += v[k]; }
      const uint32_t incl = wave_prefix_sum(sum);   // wave 0, every lane active
      uint32_t before = incl - sum;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (before < left && left <= before + v[k]) {
          sh.digit = 255 - 4 * t - k;
          sh.above = before;
          sh.bin = v[k];
        }
        before += v[k];
      }
    }
    __syncthreads();
    left -= sh.above;
    prefix |= static_cast<uint64_t>(sh.digit) << shift;
    if ((kTopK - left) + sh.bin <= kTopkSortCap) { thr = prefix; break; }
  }
  const uint32_t need = min(total, static_cast<uint32_t>(kTopK));
  __syncthreads();
  if (tid == 0) sh.count = 0;
  __syncthreads();
  for (uint32_t p0 = 0; p0 < n; p0 += kU * kTopkThreads) {
    uint64_t kk[kU];
    keys(p0, kk);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (kk[u] != 0 && kk[u] >= thr) {
        const uint32_t pos = atomicAdd(&sh.count, 1u);
        if (pos < kTopkSortCap) sh.cand[pos] = kk[u];   // at most 1024 by construction
      }
    }
  }
  __syncthreads();
  const uint32_t nk = min(sh.count, static_cast<uint32_t>(kTopkSortCap));
  if (tid >= nk) sh.cand[tid] = 0;
  __syncthreads();
  const uint32_t size = nk <= kTopK ? kTopK : kTopkSortCap;
  for (uint32_t k = 2; k <= size; k <<= 1) {
    for (uint32_t j = k >> 1; j > 0; j >>= 1) {
      const uint32_t ixj = tid ^ j;
      if (tid < size && ixj > tid) {
        const uint64_t x = sh.cand[tid], y = sh.cand[ixj];
        const bool desc = (tid & k) == 0;
        if (desc ? (x < y) : (x > y)) { sh.cand[tid] = y; sh.cand[ixj] = x; }
      }
      __syncthreads();
    }
  }
  if (tid < kTopK) emit(tid, tid < need ? sh.cand[tid] : 0ull);
}

// One row's arguments of a selection level. They are read in one batch at
// the start of the kernel: the level's first loads (candidates, floors)
// depend on several of them, and read one by one they cost a chain of
// dependent scalar-load round trips.
struct LevelRow {
  const uint64_t *in;        // the row's input lists (later levels)
  const float *scores;       // the row's scores
  const uint64_t *floors;    // the row's wave floors (checked final level)
  uint64_t *out;             // the row's output lists (levels before the final one)
  uint32_t count;            // candidates of the row at this level
  uint32_t floor_count;
  uint32_t fallback_count;   // scores to select from when the check fails
  int32_t offset;
  bool final_level;
  bool check;                // final level over fused-indexer candidates: check the floors
};

// Row r's LevelRow. x0 and x1 are two more 32-bit arguments of the caller,
// read in the same batch (each goes in as a value read from the arguments and
// comes out unchanged).
__device__ __forceinline__ LevelRow level_row(const TopkLevelArgs &a, uint32_t r, uint32_t &x0, uint32_t &x1) {
  uint64_t in = reinterpret_cast<uint64_t>(a.in), in_base = a.in_base[r];
  uint64_t sc = reinterpret_cast<uint64_t>(a.scores), stride = a.score_stride;
  uint64_t fl = reinterpret_cast<uint64_t>(a.floors);
  uint64_t out = reinterpret_cast<uint64_t>(a.out), out_base = a.out_base[r];
  uint32_t floor_begin = a.floor_begin[r];
  uint32_t count = a.count[r], fc = a.floor_count[r], fb = a.fallback_count[r];
  uint32_t off = static_cast<uint32_t>(a.offset[r]);
  uint32_t fmask = a.final_mask, cmask = a.check_mask;
  // One use of every loaded value, before any arithmetic on them: the scalar
  // loads issue together, with one wait.
  asm volatile("" : "+s"(in), "+s"(in_base), "+s"(sc), "+s"(stride), "+s"(fl), "+s"(out), "+s"(out_base),
               "+s"(floor_begin), "+s"(count), "+s"(fc), "+s"(fb), "+s"(off), "+s"(fmask), "+s"(cmask), "+s"(x0),
               "+s"(x1));
  LevelRow lr;
  lr.in = global_ptr<const uint64_t>(in) + in_base;
  lr.scores = global_ptr<const float>(sc) + r * stride;
  lr.floors = global_ptr<const uint64_t>(fl) + floor_begin;
  lr.out = global_ptr<uint64_t>(out) + out_base;
  lr.count = count;
  lr.floor_count = fc;
  lr.fallback_count = fb;
  lr.offset = static_cast<int32_t>(off);
  lr.final_level = ((fmask >> r) & 1u) != 0;
  lr.check = lr.final_level && ((cmask >> r) & 1u) != 0;
  return lr;
}

// One workgroup's selection over chunk `chunk` of row r (one top-k level).
// kFromScores: the first level, reading f32 scores. Otherwise a later level,
// reading the previous level's 64-bit key lists.
// kPer: candidates per thread, so that a chunk holds 1024 kPer of them: on
// the first level 32, or 4, 8 or 16 when every row of the level fits one
// such chunk (short rows: less work per thread); on later levels 8, or 4
// when every row of the level has at most 4096.
// emit_final(pos, index): the final level's index of rank pos (index +
// offset, or -1 for an empty slot).
// A caller that has already loaded the level's candidates (kFromScores
// false, chunk 0: candidate e of this thread at position tid + 1024 e, from
// anywhere in the row's room) passes them as pre_keys with have_pre set, and
// likewise the floor at position min(tid, room - 1) as pre_floor with
// have_pre_floor set; positions past the row's own count are masked here.
template <bool kFromScores, int kPer, class EmitFinal>
__device__ __forceinline__ void select_level(TopkShared &sh, const LevelRow &lr, uint32_t chunk,
                                             const EmitFinal &emit_final, bool have_pre,
                                             const uint64_t (&pre_keys)[kPer], bool have_pre_floor,
                                             uint64_t pre_floor) {
  static_assert(kPer <= kTopkPerThreadFirst, "the first level's LDS holds 32 score slots per thread");
  constexpr uint32_t kChunk = kTopkThreads * kPer;

  const uint32_t begin = chunk * kChunk;
  const uint32_t end = min(lr.count, begin + kChunk);
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, known to the compiler
  const bool final_level = lr.final_level;

  sh.hist[tid] = 0;
  sh.cursor[tid] = 0;
  if (tid == 0) {
    sh.count = 0;
    sh.lo = 0;
    sh.viol = 0;
    sh.s_total = 0;
    sh.s_min1 = 0xFFFFFFFFu;
    sh.s_max = 0;
    sh.s_floor = 0;
  }

  // Candidate e of this thread sits at position begin + tid + 1024 * e.
  // Loads are unconditional, from positions clamped into the row (every row
  // holds at least one score or list entry), and masked afterwards: loads
  // under a branch would make the compiler wait for each one in turn. Each
  // load takes a uniform base and a 32-bit byte offset (rows hold < 2^30
  // entries), so it needs one offset register rather than a 64-bit address.
  const uint32_t lastp = end > 0 ? end - 1 : 0;
  uint32_t ordv[kFromScores ? kPer : 1];     // score bits, 0 = no candidate
  uint64_t keyv[kFromScores ? 1 : kPer];
  if constexpr (kFromScores) {
    const char *sc = reinterpret_cast<const char *>(lr.scores);
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      ordv[e] = *reinterpret_cast<const uint32_t *>(sc + 4u * min(begin + tid + kTopkThreads * e, lastp));
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint32_t p = begin + tid + kTopkThreads * e;
      ordv[e] = p < end ? static_cast<uint32_t>(topk_key(__uint_as_float(ordv[e]), p) >> 32) : 0u;
    }
  } else {
    if (have_pre) {   // uniform
#pragma unroll
      for (int e = 0; e < kPer; ++e) keyv[e] = pre_keys[e];
    } else {
      const char *in = reinterpret_cast<const char *>(lr.in);
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        keyv[e] = *reinterpret_cast<const uint64_t *>(in + 8u * min(begin + tid + kTopkThreads * e, lastp));
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if (begin + tid + kTopkThreads * e >= end) keyv[e] = 0;
  }
  // A checked final level compares the row's highest floor with the last
  // selected key; the floors are loaded now, with the candidates.
  const bool check_row = !kFromScores && lr.check;
  uint64_t floor_hi = 0;
  if constexpr (!kFromScores) {
    if (check_row && lr.floor_count > 0) {
      // (A prefetched floor past the row's own floors is not one of them: 0.)
      floor_hi = have_pre_floor ? (tid < lr.floor_count ? pre_floor : 0ull) : lr.floors[min(tid, lr.floor_count - 1)];
      for (uint32_t b = tid + kTopkThreads; b < lr.floor_count; b += kTopkThreads) floor_hi = max(floor_hi, lr.floors[b]);
    }
  }
  // The statistics' starting values are in place before any wave adds to
  // them (the waves pass this barrier while their loads are in flight).
  __syncthreads();
  auto run = [&](const auto &c) {
    // Count and extreme score bits of the valid keys. A missing key has high
    // word 0 (every valid key's is nonzero), so it never raises the maximum
    // and, as 0 - 1 in unsigned arithmetic, never lowers the minimum. The
    // count comes from one ballot per candidate slot (scalar popcounts); the
    // extremes from lane reductions. Sixteen waves share the CU's four SIMDs
    // here, so every vector instruction of this phase is paid four times.
    uint32_t nvalid = 0, omin1 = 0xFFFFFFFFu, omax = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint32_t o = c.hi(e);
      nvalid += static_cast<uint32_t>(__popcll(__ballot(o != 0)));
      omin1 = min(omin1, o - 1u);
      omax = max(omax, o);
    }
    // Per-wave totals, combined across the waves by one LDS atomic per
    // statistic from each wave; every thread reads the four results after a
    // barrier (combining sixteen per-wave slots in every thread cost more
    // than the rest of this phase). The reduced values are made explicitly
    // wave-uniform, so that each atomic is a single instruction rather than
    // the compiler's loop over the active lanes.
    omin1 = __builtin_amdgcn_readfirstlane(wave_min(omin1));
    omax = __builtin_amdgcn_readfirstlane(wave_max(omax));
    // Only the waves holding floors (threads below floor_count) reduce them;
    // the others' floors are all 0, the maximum's starting value.
    const bool wave_floors = check_row && wave * 64u < lr.floor_count;   // uniform
    uint64_t wfloor = 0;
    if (wave_floors) {   // 64-bit wave maximum: the high words, then the low words of the lanes holding it
      const uint32_t hi = __builtin_amdgcn_readfirstlane(wave_max(static_cast<uint32_t>(floor_hi >> 32)));
      const uint32_t lo = __builtin_amdgcn_readfirstlane(
          wave_max(static_cast<uint32_t>(floor_hi >> 32) == hi ? static_cast<uint32_t>(floor_hi) : 0u));
      wfloor = (static_cast<uint64_t>(hi) << 32) | lo;
    }
    if (lane == 0) {
      atomicAdd(&sh.s_total, nvalid);
      atomicMin(&sh.s_min1, omin1);
      atomicMax(&sh.s_max, omax);
      if (wave_floors) atomicMax(reinterpret_cast<unsigned long long *>(&sh.s_floor), static_cast<unsigned long long>(wfloor));
    }
    __syncthreads();
    const uint32_t total = sh.s_total, min1 = sh.s_min1, gmax = sh.s_max;
    const uint64_t max_floor = sh.s_floor;
    const uint32_t need = min(total, static_cast<uint32_t>(kTopK));
    const uint32_t gmin = min1 + 1u;

    // A checked final level writes its result as it goes: a key that a wave
    // of the fused indexer did not write ranks below that wave's floor key,
    // so the result stands unless the row's highest floor lies above the last
    // selected key (or the row has fewer than 512 candidates and some wave
    // left keys out); then the row is selected again from its scores, which
    // rewrites every slot. (Fused-indexer candidates are lists, so only later
    // levels check.)
    const bool check = check_row;
    auto emit_out = [&](uint32_t pos, uint64_t kk) {
      if (final_level) {
        emit_final(pos, kk != 0 ? static_cast<int32_t>(~static_cast<uint32_t>(kk)) + lr.offset : -1);
      } else {
        lr.out[static_cast<uint64_t>(chunk) * kTopK + pos] = kk;
      }
    };
    auto emit = [&](uint32_t pos, uint64_t kk) {
      emit_out(pos, kk);
      if (check && pos + 1 == static_cast<uint32_t>(kTopK) && max_floor > kk)
        sh.viol = 1;
    };
    // Best `need` of this chunk's candidates (total valid, score bits in
    // [gmin, gmax]), in rank order through emit(pos, key).
    auto select_chunk = [&](uint32_t total, uint32_t need, uint32_t gmin, uint32_t gmax, const auto &emit) {
      // Threshold T from the sample (every key when the chunk is small).
      uint32_t thr = 1;
      const bool sampled = end - begin > kSmallChunk;
      if (sampled) {
        const float smin = ord_score(gmin), smax = ord_score(gmax);
        const float range = smax - smin;
        const float scale = (range > 0.0f && __builtin_isfinite(range)) ? static_cast<float>(kBins) / range : 0.0f;
        const uint32_t o0 = c.hi(0);
        const uint32_t b0 = o0 != 0 ? static_cast<uint32_t>(fminf((ord_score(o0) - smin) * scale,
                                                                   static_cast<float>(kBins - 1)))
                                    : static_cast<uint32_t>(kBins);
        hist_add(sh.hist, b0, kBins, lane);
        __syncthreads();
        uint32_t h, above, maxge, nsamp;
        scan_bins(sh.hist, sh.wsum, sh.wmax, tid, h, above, maxge, nsamp);
        const uint32_t target = sample_target<kPer>(nsamp);
        if (target > 0 && above < target && target <= above + h) sh.lo = kBins - 1 - tid;
        if (nsamp == 0 && tid == 0) sh.lo = 0;
        __syncthreads();
        const uint32_t lo = sh.lo;
        // T: the score bits of the lower edge of bin lo - 1, one bin below
        // the sampled bin, so that the keys binned at lo or above (about the
        // sample's share) are kept with a few more; lo = 0 (also a zero
        // range) keeps every valid key. Whatever T is, the keys at or above
        // it are the best ones in score order: when they number at least
        // `need`, the selection over them is exact, and otherwise the path
        // below selects over every candidate.
        if (lo > 0) {
          const float edge = smin + static_cast<float>(lo - 1) / scale;
          thr = max(1u, static_cast<uint32_t>(topk_key(edge, 0) >> 32));
        }
      }
      if constexpr (!kFromScores) {
        if (!sampled) {
          // Every valid key stays: select over the candidates as loaded, on
          // the shared arrays as the kernel initialised them.
          counting_select<kPer, false, true, true>(sh, c, total, need, gmin, gmax, emit);
          return;
        }
      }
      // Compaction: keys with score bits >= T go to the wave's region, in
      // candidate order; the running count is wave-uniform.
      uint64_t *region = sh.compact + wave * kCompactPerWave;
      uint32_t wcount = 0;
  #pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const bool in = c.hi(e) >= thr;            // a missing key (0) is below any T >= 1
        const uint64_t mask = __ballot(in);
        const uint32_t pos = wcount + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
        if (in && pos < kCompactPerWave) region[pos] = c.vkey(e);
        wcount += static_cast<uint32_t>(__popcll(mask));
      }
      if (lane == 0) sh.wcount[wave] = wcount;
      __syncthreads();
      uint32_t kept = 0, overflow = 0;
  #pragma unroll
      for (int v = 0; v < kWaves / 4; ++v) {
        const u32x4 w4 = reinterpret_cast<const u32x4 *>(sh.wcount)[v];
  #pragma unroll
        for (int k = 0; k < 4; ++k) {
          kept += w4[k];
          overflow |= w4[k] > kCompactPerWave ? 1u : 0u;
        }
      }
      if (!overflow && kept >= need) {
        // The chunk's best keys are the best of the kept ones.
        uint64_t kc[kCompactPerLane];
  #pragma unroll
        for (int j = 0; j < kCompactPerLane; ++j)
          kc[j] = lane + 64u * j < wcount ? region[lane + 64 * j] : 0ull;
        counting_select<kCompactPerLane, false, false, !kFromScores>(sh, KeyCand<kCompactPerLane>{kc}, kept, need,
                                                                     max(thr, gmin), gmax, emit);
      } else if constexpr (kFromScores) {
        // Heavy ties: select over every candidate. The score bits move to LDS
        // (over the compaction regions), which frees their registers.
        __syncthreads();
  #pragma unroll
        for (int e = 0; e < kPer; ++e) sh.ordl[tid + kTopkThreads * e] = c.hi(e);
        counting_select<kPer, true>(sh, LdsOrdCand{sh.ordl, tid, begin + tid}, total, need, gmin, gmax, emit);
      } else {
        counting_select<kPer, true>(sh, c, total, need, gmin, gmax, emit);
      }
    };
    // Slots past the selected count are empty.
    for (uint32_t t = need + tid; t < kTopK; t += kTopkThreads) emit(t, 0);
    if (total > 0) select_chunk(total, need, gmin, gmax, emit);
    if constexpr (kFromScores) return;
    if (!check) return;
    __syncthreads();   // the last rank's verdict (viol was cleared at the start)
    if ((need < static_cast<uint32_t>(kTopK) && max_floor != 0) || sh.viol != 0) {   // uniform
      // The output stores of every wave land before the second barrier, so
      // that the reselection rewrites them rather than racing them (on the
      // common path nothing waits for them).
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      __syncthreads();
      select_from_scores(sh, lr.scores, lr.fallback_count, emit_out);
    }
  };
  if constexpr (kFromScores) run(OrdCand<kPer>{ordv, begin + tid});
  else run(KeyCand<kPer>{keyv});
}
// The same, loading the candidates and floors itself.
template <bool kFromScores, int kPer, class EmitFinal>
__device__ __forceinline__ void select_level(TopkShared &sh, const LevelRow &lr, uint32_t chunk,
                                             const EmitFinal &emit_final) {
  const uint64_t none[kPer] = {};
  select_level<kFromScores, kPer>(sh, lr, chunk, emit_final, false, none, false, 0ull);
}

}  // namespace ds
