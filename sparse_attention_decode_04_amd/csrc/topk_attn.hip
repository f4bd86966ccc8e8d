// A row's final top-k level and its sparse attention in one kernel.
//
// What is computed is exactly ds_rows_indexer_topk's last level (the best 512
// of the fused indexer's candidates in rank order, checked against the
// waves' floors, with the reselection from scores when a floor could hide a
// ranking key) followed by phase 1 of ds_rows_sparse_attn_direct on those
// indices. Sources: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernels deepseek_indexer_topk_finalize_rows_i32 (the final indices) and
// deepseek_sparse_attention_score_rows_bf16 (the attention reading the KV
// through them); "mlx-native 0.21.0 src/ops/deepseek_rows.rs", the rows
// dispatches that run them back to back.
//
// Mapping: one 1024-thread workgroup per (row, group of 16 heads, 64-slot
// chunk), as many as the attention has. Every workgroup runs its row's
// selection itself (the row's 32 workgroups repeat it, each on its own CU,
// where one workgroup per row would leave the chunks waiting for a kernel
// boundary) and keeps the indices of its own 64 slots in LDS; the
// workgroups of head group 0 also write their slots to the index output (the
// last chunk's also the slots past the row's width).
// The selection's LDS is then reused for the chunk's attention, which all
// sixteen waves compute as the attention kernel does, its indices read
// from LDS instead of memory. This removes a kernel boundary and the
// attention's dependent index load (two HBM round trips become one).
#include "attn_chunk.hpp"
#include "topk_select.hpp"

namespace ds {

template <int kPerLater>
__global__ __launch_bounds__(kTopkThreads) void topk_attn_kernel(TopkLevelArgs t, AttnArgs a) {
  __shared__ union Shared {
    TopkShared sel;
    AttnChunkShared att;
  } u;
  __shared__ int32_t slot_index[kAttnChunk];

  // Row r on XCD r, as in the attention kernel.
  const uint32_t r = blockIdx.x % kXcds;
  const uint32_t rest = blockIdx.x / kXcds;
  const uint32_t hg = rest % kAttnHeadGroups;
  const uint32_t c = rest / kAttnHeadGroups;
  uint32_t rows = a.rows, chunks = a.chunks[r];
  const LevelRow lr = level_row(t, r, rows, chunks);   // one batch of argument loads
  if (r >= rows || c >= chunks) return;   // uniform
  const uint32_t lo = c * kAttnChunk;
  // Head group 0 writes the index output: each chunk its own 64 slots, the
  // last chunk also every slot past the row's width.
  const uint32_t out_end = c + 1 == chunks ? static_cast<uint32_t>(kTopK) : lo + kAttnChunk;
  int32_t *const out = t.indices + t.out_offset[r];
  select_level<false, kPerLater>(u.sel, lr, 0, [&](uint32_t pos, int32_t index) {
    if (pos - lo < static_cast<uint32_t>(kAttnChunk)) slot_index[pos - lo] = index;   // pos in [lo, lo + 64)
    if (hg == 0 && pos >= lo && pos < out_end) out[pos] = index;
  });
  __syncthreads();   // the chunk's indices are in place; the selection's LDS is free
  uint64_t unused64 = 0;
  uint32_t unused32 = 0;
  const AttnRow ar = attn_row<true>(a, r, rows, chunks, unused64, unused32);
  static_assert(kTopkThreads == kChunkThreads, "the attention chunk uses every thread of the workgroup");
  attn_chunk_body<true>(u.att, ar, hg, c, [&](uint32_t slot) { return slot_index[slot - lo]; });
}

hipError_t launch_topk_attn(const TopkLevelArgs &t, const AttnArgs &a, uint32_t blocks, hipStream_t s) {
  if (t.per_thread == 4)
    hipLaunchKernelGGL(topk_attn_kernel<4>, dim3(blocks), dim3(kTopkThreads), 0, s, t, a);
  else
    hipLaunchKernelGGL(topk_attn_kernel<kTopkPerThreadLater>, dim3(blocks), dim3(kTopkThreads), 0, s, t, a);
  return hipGetLastError();
}

}  // namespace ds
