// Deterministic causal top-512 of each row's indexer scores.
//
// Order (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// index_rows_better): keys without a finite score or past the causal limit
// never rank; otherwise the higher score ranks first and equal scores rank by
// the lower index. The pages compute it with a 1024-key bitonic block sort
// (deepseek_indexer_topk_block_rows_i32), a pairwise merge-path tree with one
// launch per round (deepseek_indexer_topk_merge_rows_i32) and a finalize pass
// (deepseek_indexer_topk_finalize_rows_i32). The result is unique (the order
// is strict and total), so this build reaches it differently:
//
//   * Every candidate becomes one 64-bit key
//       (order-preserving bits of (score + 0.0f)) << 32 | ~index
//     so that unsigned key order is exactly the pages' order (+0.0f folds -0
//     into +0, which the pages' float comparison treats as equal) and 0 means
//     "no candidate".
//   * One level: each 1024-thread workgroup takes up to 8192 candidates of one
//     row, finds a threshold by MSB-first 8-bit radix select on the keys (an
//     LDS histogram per digit, wave-aggregated when a wave's digits agree),
//     stops as soon as at most 1024 keys lie at or above the candidate prefix,
//     compacts those into LDS, sorts them with a bitonic network and keeps the
//     best 512 in order.
//   * Levels repeat on the 512-key lists until each row has one list; the
//     last level writes index + offset, or -1 for empty slots. A row of n
//     visible keys needs ceil(log_16(n/512)) levels: one up to 8192 keys, two
//     up to 131072, three up to 2M.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

__device__ __forceinline__ uint64_t topk_key(float s, uint32_t index) {
  if (!__builtin_isfinite(s)) return 0;
  s += 0.0f;                                   // -0 -> +0
  const uint32_t u = __float_as_uint(s);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~index);
}

__global__ __launch_bounds__(kTopkThreads) void topk_level_kernel(TopkLevelArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint64_t cand[kTopkSortCap];
  __shared__ uint32_t s_valid, s_count, s_digit, s_above, s_bin;

  const uint32_t r = row_of_block(a.blk_begin, blockIdx.x);
  const uint32_t chunk = blockIdx.x - a.blk_begin[r];
  const uint32_t begin = chunk * kTopkChunk;
  const uint32_t end = min(a.count[r], begin + kTopkChunk);
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;

  if (tid == 0) { s_valid = 0; s_count = 0; }

  // Candidate e of this thread sits at position begin + tid + 1024 * e.
  uint64_t key[kTopkPerThread];
  if (a.from_scores) {
    const float *sc = a.scores + static_cast<uint64_t>(r) * a.score_stride;
#pragma unroll
    for (int e = 0; e < kTopkPerThread; ++e) {
      const uint32_t p = begin + tid + kTopkThreads * e;
      key[e] = p < end ? topk_key(sc[p], p) : 0;
    }
  } else {
    const uint64_t *in = a.in + a.in_base[r];
#pragma unroll
    for (int e = 0; e < kTopkPerThread; ++e) {
      const uint32_t p = begin + tid + kTopkThreads * e;
      key[e] = p < end ? in[p] : 0;
    }
  }
  __syncthreads();

  uint32_t nvalid = 0;
#pragma unroll
  for (int e = 0; e < kTopkPerThread; ++e) nvalid += __popcll(__ballot(key[e] != 0));
  if (lane == 0) atomicAdd(&s_valid, nvalid);
  __syncthreads();
  const uint32_t total = s_valid;

  // Threshold: keep keys >= thr. With at most kTopkSortCap candidates keep
  // them all; otherwise radix-select digits until the kept set is small.
  uint64_t thr = 1;
  if (total > kTopkSortCap) {
    uint32_t need = kTopK;          // ranks still to fill below the prefix
    uint64_t prefix = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kTopkPerThread; ++e) {
        const bool match = key[e] != 0 &&
                           (shift == 56 || (key[e] >> (shift + 8)) == (prefix >> (shift + 8)));
        const uint32_t dig = match ? static_cast<uint32_t>(key[e] >> shift) & 255u : 256u;
        const uint32_t first = __builtin_amdgcn_readfirstlane(dig);
        const uint64_t same = __ballot(dig == first);
        if (same == __ballot(true)) {
          if (first != 256u && lane == 0) atomicAdd(&hist[first], static_cast<uint32_t>(__popcll(same)));
        } else if (dig != 256u) {
          atomicAdd(&hist[dig], 1u);
        }
      }
      __syncthreads();
      if (tid < 64) {
        // Lane l holds bins 255-4l .. 252-4l (descending). Find the bin where
        // the count of keys ranked above it first reaches `need`.
        uint32_t v[4], sum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) { v[k] = hist[255 - 4 * tid - k]; sum += v[k]; }
        uint32_t incl = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t up = __shfl_up(incl, o);
          if (tid >= static_cast<uint32_t>(o)) incl += up;
        }
        uint32_t before = incl - sum;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (before < need && need <= before + v[k]) {
            s_digit = 255 - 4 * tid - k;
            s_above = before;
            s_bin = v[k];
          }
          before += v[k];
        }
      }
      __syncthreads();
      const uint32_t digit = s_digit;
      need -= s_above;
      prefix |= static_cast<uint64_t>(digit) << shift;
      const uint32_t kept = (kTopK - need) + s_bin;
      __syncthreads();   // s_* and hist are rewritten by the next pass
      if (kept <= kTopkSortCap) { thr = prefix; break; }
    }
  }

  // Compact the kept keys (order arbitrary; sorted next).
#pragma unroll
  for (int e = 0; e < kTopkPerThread; ++e) {
    if (key[e] != 0 && key[e] >= thr) {
      const uint32_t pos = atomicAdd(&s_count, 1u);
      if (pos < kTopkSortCap) cand[pos] = key[e];   // at most 1024 by construction
    }
  }
  __syncthreads();
  const uint32_t kept = min(s_count, static_cast<uint32_t>(kTopkSortCap));
  for (uint32_t i = tid; i < kTopkSortCap; i += kTopkThreads)
    if (i >= kept) cand[i] = 0;
  __syncthreads();

  // Bitonic sort, descending, over the smallest power of two >= 512 covering
  // the kept keys.
  const uint32_t size = kept <= kTopK ? kTopK : kTopkSortCap;
  for (uint32_t k = 2; k <= size; k <<= 1) {
    for (uint32_t j = k >> 1; j > 0; j >>= 1) {
      const uint32_t ixj = tid ^ j;
      if (tid < size && ixj > tid) {
        const uint64_t x = cand[tid], y = cand[ixj];
        const bool desc = (tid & k) == 0;
        if (desc ? (x < y) : (x > y)) { cand[tid] = y; cand[ixj] = x; }
      }
      __syncthreads();
    }
  }

  if (tid < kTopK) {
    const uint64_t kk = cand[tid];
    if ((a.final_mask >> r) & 1u) {
      const int32_t idx = kk != 0 ? static_cast<int32_t>(~static_cast<uint32_t>(kk)) + a.offset[r] : -1;
      a.indices[a.out_offset[r] + tid] = idx;
    } else {
      a.out[a.out_base[r] + static_cast<uint64_t>(chunk) * kTopK + tid] = kk;
    }
  }
}

hipError_t launch_topk_level(const TopkLevelArgs &a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(topk_level_kernel, dim3(blocks), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
