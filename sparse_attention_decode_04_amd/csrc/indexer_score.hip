// Lightning-indexer score of one query per row, bf16 MFMA on gfx950.
//
// Computes, for key j of row r,
//   s[j] = sum_h w[h] * max(0, sum_d q[h,d] * k[j,d])      (64 heads, d < 128)
// and stores -inf for keys at or past the causal limit or with a non-finite
// score. Source: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernel deepseek_indexer_score_mma_rows_bf16 (score, ReLU, head-weight
// epilogue, causal mask, finite check).
//
// Mapping (differs from the pages' Metal design: no threadgroup staging, no
// fp16 conversion; bf16 products are exact in the f32 accumulator):
//   * MFMA 16x16x32 with M = 16 heads, N = 16 keys, K = 32 features; four
//     head tiles x four feature steps per 16-key tile.
//   * Lane l of a wave serves key l%16 and the 64 contiguous bytes
//     [64*(l/16), +64) of that key's 256-byte row: feature step c uses bytes
//     16c of that span. The query fragments are loaded with the same feature
//     assignment, so the contraction is unchanged.
//   * D lane l holds heads 16m + 4*(l/16) + i of key l%16: the ReLU and head
//     weights are applied in registers, then two cross-lane adds finish the
//     head sum.
//   * The query (64 x 128 bf16) stays in 64 VGPRs for the wave's lifetime;
//     key tiles are double-buffered in registers so the next tile's four
//     16-byte loads are in flight while the current tile's 16 MFMAs run.
// The arithmetic per key is a fixed instruction sequence independent of the
// row count or of other rows, so every row is bitwise identical to a
// one-row launch.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

__global__ __launch_bounds__(kIdxThreads) void indexer_score_kernel(IndexerArgs a) {
  const uint32_t r = row_of_block(a.blk_begin, blockIdx.x);
  const uint32_t n = a.kv_len[r];
  const uint32_t visible = a.visible[r];
  const uint32_t k0 = (blockIdx.x - a.blk_begin[r]) * a.keys_per_block;
  const uint32_t k_end = min(n, k0 + a.keys_per_block);
  const uint16_t *__restrict__ keys = a.keys[r];
  const uint16_t *__restrict__ q = a.q + static_cast<uint64_t>(a.q_row[r]) * kHeads * kIdxDim;
  const float *__restrict__ w = a.w + static_cast<uint64_t>(a.q_row[r]) * kHeads;
  float *__restrict__ scores = a.scores + static_cast<uint64_t>(r) * a.score_stride;

  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t col = lane & 15;   // key within tile / head within head tile
  const uint32_t grp = lane >> 4;   // 64-byte span of the 256-byte row

  // Query fragments: head 16m + col, features [32*grp + 8c, +8).
  bf16x8 qa[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint16_t *qrow = q + (16 * m + col) * kIdxDim + 32 * grp;
#pragma unroll
    for (int c = 0; c < 4; ++c) qa[m][c] = as_bf16x8(load16(qrow + 8 * c));
  }
  // Head weights of the D rows this lane holds.
  float wt[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) wt[m][i] = w[16 * m + 4 * grp + i];

  const uint32_t tiles = (k_end - k0 + kIdxTile - 1) / kIdxTile;
  uint32_t t = wave;
  if (t >= tiles) return;

  auto load_tile = [&](uint32_t tile, u32x4 (&kb)[4]) {
    const uint32_t key = min(k0 + tile * kIdxTile + col, n - 1);   // tail: clamp, not stored
    const uint16_t *krow = keys + static_cast<uint64_t>(key) * kIdxDim + 32 * grp;
#pragma unroll
    for (int c = 0; c < 4; ++c) kb[c] = load16(krow + 8 * c);
  };

  u32x4 cur[4], nxt[4];
  load_tile(t, cur);
  for (; t < tiles; t += 4) {
    const bool more = t + 4 < tiles;
    if (more) load_tile(t + 4, nxt);

    float part = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma16(qa[m][c], as_bf16x8(cur[c]), acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) part = fmaf(fmaxf(acc[i], 0.0f), wt[m][i], part);
    }
    // Sum the four 16-head groups held by lanes col, col+16, col+32, col+48.
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);

    const uint32_t key = k0 + t * kIdxTile + col;
    if (grp == 0 && key < k_end) {
      scores[key] = (key < visible && __builtin_isfinite(part)) ? part : -__builtin_inff();
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < 4; ++c) cur[c] = nxt[c];
    }
  }
}

hipError_t launch_indexer_score(const IndexerArgs &a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(indexer_score_kernel, dim3(blocks), dim3(kIdxThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
