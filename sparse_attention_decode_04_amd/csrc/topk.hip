// Deterministic causal top-512 of each row's indexer scores.
//
// Order (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// index_rows_better): keys without a finite score or past the causal limit
// never rank; otherwise the higher score ranks first and equal scores rank by
// the lower index. The pages compute it with a 1024-key bitonic block sort
// (deepseek_indexer_topk_block_rows_i32), a pairwise merge-path tree with one
// launch per round (deepseek_indexer_topk_merge_rows_i32) and a finalize pass
// (deepseek_indexer_topk_finalize_rows_i32). The result is unique (the order
// is strict and total), so this build reaches it differently.
//
// Keys. Every candidate is one 64-bit key
//     (order-preserving bits of (score + 0.0f)) << 32 | ~index
// so that unsigned key order is exactly the pages' order (+0.0f folds -0 into
// +0, which the pages' float comparison treats as equal) and 0 means "none".
//
// One level. A 1024-thread workgroup takes a chunk of one row's candidates,
// held in registers (first level: 32768 scores, 32 per thread, kept as their
// 32 score bits; later levels: 8192 list keys, 8 per thread), and writes that
// chunk's best min(512, n) keys in rank order.
//   Threshold and compaction (common case). A sample (each thread's first key)
//   gives a threshold T: the smallest sampled score in the top bins holding 64
//   of the 1024 samples. Every key >= T is appended, by one compare and a
//   ballot per key, to its wave's LDS region (512 keys per wave). When no
//   region overflows and at least min(512, n) keys were kept, the chunk's best
//   keys are exactly the best keys of that set of a few thousand, which the
//   counting select below then orders with 8 keys per thread. Chunks of at
//   most 4096 candidates keep every key.
//   Counting select: with smin/smax the extreme scores of the candidates,
//   bin(s) = min(1023, floor((s - smin) * 1024 / (smax - smin))) is monotone
//   in the score and equal scores share a bin, so every key in a higher bin
//   outranks every key in a lower one. One LDS histogram (keys of bins >= a
//   sampled lower bin when the candidates are many) and one block scan give
//   the bin d holding the 512th key and every bin's suffix count; keys of bins
//   >= d are scattered into LDS grouped by bin, and a key's rank is its bin's
//   suffix count plus the number of larger keys in its own bin. Taken when at
//   most 1024 keys lie in bins >= d and no such bin holds more than 64 keys.
//   Fallback (heavy ties, extreme outliers): MSB-first 8-bit radix select on
//   the 64-bit keys until at most 1024 remain at or above the prefix, then a
//   bitonic sort of those in LDS.
//   When the compaction does not hold (heavy ties), the counting select runs
//   on all of the chunk's candidates instead.
// The code that runs in the common case is kept short: on this GPU a kernel
// pays for every cold instruction-cache line it executes.
// Levels repeat on the lists until each row has one; the last level writes
// index + offset, or -1 for empty slots. A row of n visible keys needs one
// level up to 32768 keys, two up to 1M (the second takes its up to 32 lists
// whole) and three beyond.
#include "topk_select.hpp"

namespace ds {

template <bool kFromScores, int kPerLater = kTopkPerThreadLater>
__global__ __launch_bounds__(kTopkThreads) void topk_level_kernel(TopkLevelArgs a) {
  __shared__ TopkShared sh;
  const uint32_t r = row_of_block(a.blk_begin, blockIdx.x);
  uint32_t blk0 = a.blk_begin[r], out_offset = a.out_offset[r];
  const LevelRow lr = level_row(a, r, blk0, out_offset);
  int32_t *const indices = a.indices + out_offset;
  select_level<kFromScores, kPerLater>(sh, lr, blockIdx.x - blk0, [&](uint32_t pos, int32_t index) { indices[pos] = index; });
}

hipError_t launch_topk_level(const TopkLevelArgs &a, uint32_t blocks, hipStream_t s) {
  if (a.from_scores) {
    if (a.per_thread == 4)
      hipLaunchKernelGGL((topk_level_kernel<true, 4>), dim3(blocks), dim3(kTopkThreads), 0, s, a);
    else if (a.per_thread == 8)
      hipLaunchKernelGGL((topk_level_kernel<true, 8>), dim3(blocks), dim3(kTopkThreads), 0, s, a);
    else if (a.per_thread == 16)
      hipLaunchKernelGGL((topk_level_kernel<true, 16>), dim3(blocks), dim3(kTopkThreads), 0, s, a);
    else
      hipLaunchKernelGGL((topk_level_kernel<true, kTopkPerThreadFirst>), dim3(blocks), dim3(kTopkThreads), 0, s, a);
  } else if (a.per_thread == 4)
    hipLaunchKernelGGL((topk_level_kernel<false, 4>), dim3(blocks), dim3(kTopkThreads), 0, s, a);
  else if (a.per_thread == 16)
    hipLaunchKernelGGL((topk_level_kernel<false, 16>), dim3(blocks), dim3(kTopkThreads), 0, s, a);
  else
    hipLaunchKernelGGL(topk_level_kernel<false>, dim3(blocks), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
