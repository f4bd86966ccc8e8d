// Sparse MQA attention over the selected KV rows (keys = values) with a
// learned per-head sink, bf16 MFMA with f32 accumulation on gfx950.
//
// What is computed (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernels deepseek_sparse_attention_score_rows_bf16 and
// deepseek_sparse_attention_reduce_rows_bf16, and the gather semantics of
// deepseek_sparse_attention_gather_rows_bf16; keys = values and one sink
// vector for every row per "mlx-native 0.21.0 src/ops/deepseek_rows.rs",
// dispatch_deepseek_sparse_attention_flash_rows):
//   l[h,t] = scale * q[h] . G[t]                   (live slots only)
//   m = max(sink[h], max_t l), Z = e^(sink-m) + sum_t e^(l-m)
//   out[h] = sum_t e^(l-m)/Z * G[t]
// with the pages' fail-closed rule: a row with a bad slot (bad index or a
// non-finite KV element; the gathered variant has the gather's per-row
// invalid flag), a head whose sink or any live logit is not finite, or a
// denominator outside (0, inf) is written as zeros; other non-finite outputs
// are zeroed. The gathered variant adds the mask entry of each slot it keeps
// (mask not -inf) to the slot's logit, as an additive attention mask.
//
// Two launches (split over the selected slots, then a combine). The selected
// rows G[t] come either from the gathered operand and its mask (after
// ds_rows_gather) or, in the direct variant, straight from each row's KV
// through the indices (the gather fused in).
//   phase 1, per (row, 64-slot chunk c, group of 16 heads), 16 waves: the
//     group's query heads (16 KiB) and the chunk's rows (64 KiB) are loaded
//     once each, into LDS (the four head groups of a chunk run on one XCD
//     and share the rows through its L2); the logits on MFMA 16x16x32
//     (M = 16 heads, N = 16 slots, K = 32 features; sixteen waves, each one
//     slot tile and a quarter of the features). Per head (one wave each):
//     the chunk max m_c,
//     p~ = exp(l - m_c) as a bf16 pair (hi = bf16(p~), lo = bf16(p~ - hi):
//     ~16 significant bits) and s_c = sum p~. Then the chunk's output
//     O_c = p~ . G_c (16 heads x 512 features, f32) on MFMA 16x16x32
//     (M = 16 heads, N = 16 features, K = 32 slots), each wave owning 32
//     features. The chunk's rows stay in LDS as loaded (slot-major); the B
//     operand, 8 consecutive slots of one feature per lane, comes from two
//     transposing LDS reads (ds_read_b64_tr_b16: within each 16-lane group,
//     lane i receives the i-th 16-bit element of the 8-byte pieces that
//     lanes 4k + i/4 address, k = 0..3).
//   phase 2, per (row, 16-feature chunk), 4 waves: m, Z and the bad flag of
//     each head from the chunk statistics and the sink, then
//     out = sum_c e^(m_c - m) O_c / Z in a fixed chunk order.
// All splits depend only on the row's own width, so rows are independent
// bit for bit, and both variants give the same bits.
#include "attn_chunk.hpp"

namespace ds {

constexpr int kCombineThreads = 256;

template <bool kDirect>
__global__ __launch_bounds__(kChunkThreads) void attn_chunk_kernel(AttnArgs a) {
  __shared__ AttnChunkShared sm;
  // Grid (x, row): the four head groups of a chunk run on one XCD and read
  // the chunk's selected rows through its L2 (see attn_block).
  const uint32_t r = blockIdx.y;
  uint32_t c, hg;
  attn_block(blockIdx.x, c, hg);
  uint32_t rows = a.rows, chunks = a.chunks[r], ioff = a.index_offset[r];
  uint64_t ibits = reinterpret_cast<uint64_t>(a.indices);
  const AttnRow ar = attn_row<kDirect>(a, r, rows, chunks, ibits, ioff);   // one batch of argument loads
  if (r >= rows || c >= chunks) return;
  const int32_t *const idx = global_ptr<const int32_t>(ibits) + ioff;
  attn_chunk_body<kDirect>(sm, ar, hg, c, [&](uint32_t slot) { return idx[slot]; });
}

// ---------------------------------------------------------------- phase 2
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const float4 *stats_all, const float *opart_all,
                                                                      float *out_all, uint32_t row_chunks,
                                                                      AttnArgs a) {
  // Grid (dim chunk, row). Thread t: head t / 4, dims d0 .. d0 + 4 kVec of
  // the workgroup's kAttnDimChunk. The leading arguments arrive in scalar
  // registers (kernel-argument preloading); row r's statistics and partials
  // start at r * row_chunks chunks, so the first loads are issued at once,
  // while the row's chunk count and output row are still being read.
  constexpr int kVec = kAttnDimChunk / 4 / 4;   // f32x4 per thread
  const uint32_t r = blockIdx.y;   // < rows: one row of workgroups per table row
  // Workgroup x of a row runs on XCD x % 8 (the grid's rows are whole
  // multiples of 8 workgroups). XCD k takes the row's dim chunks 4k .. 4k + 3:
  // 64 consecutive dims, two whole 128-byte lines of every partial row, so
  // each line is fetched into one L2 only (with neighbouring chunks on
  // different XCDs every line was fetched twice, once per half).
  static_assert(kDim / kAttnDimChunk == 4 * kXcds, "four dim chunks per XCD");
  const uint32_t dc = 4 * (blockIdx.x % kXcds) + blockIdx.x / kXcds;
  const uint32_t nch = a.chunks[r], q_row = a.q_row[r];
  const uint32_t tid = threadIdx.x;
  const uint32_t head = tid >> 2;
  const uint32_t d0 = kAttnDimChunk * dc + 4 * kVec * (tid & 3);
  const float4 *stats = stats_all + static_cast<uint64_t>(r) * row_chunks * kHeads + head;
  const float *op = opart_all + (static_cast<uint64_t>(r) * row_chunks * kHeads + head) * kDim + d0;
  constexpr int kB = 8;   // chunks per batch of loads
  // Chunk c of the row (c < nch). The first batch is clamped to the row's
  // room instead, so that its loads need no argument; the chunks in
  // [nch, room) it reads hold nothing of this call and are never used:
  // every use of the first batch below is a select on c < nch.
  auto stat_at = [&](uint32_t cc) { return stats[static_cast<uint64_t>(min(cc, nch - 1)) * kHeads]; };
  auto part_at = [&](uint32_t cc, int h) {
    return *reinterpret_cast<const f32x4 *>(op + static_cast<uint64_t>(min(cc, nch - 1)) * kHeads * kDim + 4 * h);
  };
  auto room_at = [&](int i) { return static_cast<uint64_t>(min(static_cast<uint32_t>(i), row_chunks - 1)); };

  // First batch of statistics and outputs, all loads in flight at once.
  float4 x[kB];
  f32x4 pv[kB][kVec];
#pragma unroll
  for (int i = 0; i < kB; ++i) x[i] = stats[room_at(i) * kHeads];
#pragma unroll
  for (int i = 0; i < kB; ++i)
#pragma unroll
    for (int h = 0; h < kVec; ++h)
      pv[i][h] = *reinterpret_cast<const f32x4 *>(op + room_at(i) * kHeads * kDim + 4 * h);
  // Every load is issued here, before any result is used: otherwise the
  // compiler sinks the partials' loads to their first use, after the
  // statistics' arithmetic, and the workgroup waits for two memory round
  // trips one after the other. (The memory clobber keeps the loads above
  // this point; the scheduling barrier keeps that arithmetic below it.)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // m, the bad flag and Z over all chunks, with the sink (phase 1 stores the
  // head's sink with every statistic).
  float w[kB];
  const HeadNorm hn = head_norm<kB>(x[0].w, nch, [&](uint32_t cc) { return x[cc]; }, stat_at, w);

  // acc = sum_c exp(m_c - m) O_c in chunk order, over the row's chunks only
  // (selects, not branches, for the first batch).
  f32x4 acc[kVec];
#pragma unroll
  for (int h = 0; h < kVec; ++h) acc[h] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    const bool in = static_cast<uint32_t>(i) < nch;
#pragma unroll
    for (int h = 0; h < kVec; ++h)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[h][k] = in ? fmaf(w[i], pv[i][h][k], acc[h][k]) : acc[h][k];
  }
  for (uint32_t cc = kB; cc < nch; ++cc) {
    const float w = chunk_weight(stat_at(cc), hn.m);
#pragma unroll
    for (int h = 0; h < kVec; ++h) {
      const f32x4 q = part_at(cc, h);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[h][k] = fmaf(w, q[k], acc[h][k]);
    }
  }
  float *dst = out_all + (static_cast<uint64_t>(q_row) * kHeads + head) * kDim + d0;
#pragma unroll
  for (int h = 0; h < kVec; ++h) {
    f32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = head_out(acc[h][k], hn.invz, hn.bad);
    *reinterpret_cast<f32x4 *>(dst + 4 * h) = v;
  }
}

hipError_t launch_attn_chunks(const AttnArgs &a, bool direct, uint32_t max_chunks, hipStream_t s) {
  const dim3 grid(kXcds * kAttnHeadGroups * ((max_chunks + kXcds - 1) / kXcds), a.rows);
  if (direct)
    hipLaunchKernelGGL(attn_chunk_kernel<true>, grid, dim3(kChunkThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_chunk_kernel<false>, grid, dim3(kChunkThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(attn_combine_kernel, dim3(kDim / kAttnDimChunk, a.rows), dim3(kCombineThreads), 0, s,
                     static_cast<const float4 *>(a.stats), static_cast<const float *>(a.opart), a.out, a.row_chunks, a);
  return hipGetLastError();
}

}  // namespace ds
