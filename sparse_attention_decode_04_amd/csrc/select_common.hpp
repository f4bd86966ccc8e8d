// Order-preserving selection keys and an LDS histogram helper, shared by the
// top-k kernels and the fused top-k stage of the indexer.
//
// Order (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// index_rows_better): keys without a finite score never rank; otherwise the
// higher score ranks first and equal scores rank by the lower index. Every
// candidate is one 64-bit key
//     (order-preserving bits of (score + 0.0f)) << 32 | ~index
// so that unsigned key order is exactly that order (+0.0f folds -0 into +0,
// which a float comparison treats as equal) and 0 means "none".
#pragma once

#include "device_common.hpp"

namespace ds {

__device__ __forceinline__ uint64_t topk_key(float s, uint32_t index) {
  if (!__builtin_isfinite(s)) return 0;
  s += 0.0f;                                   // -0 -> +0
  const uint32_t u = __float_as_uint(s);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~index);
}

__device__ __forceinline__ float ord_score(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// LDS histogram increment by the active lanes of a wave (callers may call it
// under a branch); one atomic by the first active lane when every active lane
// has the same bin (heavy ties), one per lane otherwise. `b` >= nbins means
// "no key".
__device__ __forceinline__ void hist_add(uint32_t *hist, uint32_t b, uint32_t nbins, uint32_t lane) {
  const uint32_t first = __builtin_amdgcn_readfirstlane(b);
  const uint64_t active = __ballot(true);
  const uint64_t same = __ballot(b == first);
  if (same == active) {
    if (first < nbins && lane == static_cast<uint32_t>(__builtin_ctzll(active)))
      atomicAdd(&hist[first], static_cast<uint32_t>(__popcll(same)));
  } else if (b < nbins) {
    atomicAdd(&hist[b], 1u);
  }
}

}  // namespace ds
