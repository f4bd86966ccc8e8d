// Lightning-indexer scores of several consecutive queries per row
// (multi-query: speculative or multi-token decode), bf16 MFMA on gfx950.
//
// Query t (< query_len) of row r sits at absolute position start_pos + t and
// scores key j as
//   s[t][j] = sum_h w_t[h] * max(0, sum_d q_t[h,d] * k[j,d])   (64 heads, d < 128)
// with -inf at or past its own causal limit min(kv_len, (start_pos+t+1)/4)
// and for a non-finite score. Source: docs.rs "mlx-native 0.18.0
// src/shaders/deepseek_rows.metal", kernel deepseek_indexer_score_mma_rows_bf16
// (its query loop over a group of up to 8 query rows, each with its own
// causal count, against keys staged once per group).
//
// With Q queries per row a key is used Q times, so at Q = 8 the contraction
// does 512 flops per key byte and the MFMA units, not HBM, set the pace.
// Mapping:
//   * Workgroup of 4 waves per `keys_per_block` keys of one row. Wave w owns
//     queries w and w + 4: their 64x128 bf16 query fragments stay in VGPRs
//     (64 per query), with the head weights of the D rows each lane holds.
//   * Keys stream through LDS in chunks of 64 (16 KiB), two chunks resident:
//     every thread loads its 64 bytes of chunk c + 1 into registers while the
//     waves compute chunk c, then stores them. In LDS the sixteen 16-byte
//     pieces of key row k are permuted (piece j at slot j ^ (k mod 16)), so
//     the MFMA operand reads of 16 consecutive keys hit 16 different slots.
//   * MFMA 16x16x32 with M = 16 heads, N = 16 keys, K = 32 features: lane l
//     takes key l%16 and the 64-byte span [64*(l/16), +64) of its row, step c
//     the 16 bytes at 16c of it; the query fragments use the same feature
//     assignment. ReLU and head weights are applied in registers and two
//     cross-lane adds finish the head sum: the per-key arithmetic is that of
//     the single-query indexer, so query_len = 1 gives its bits.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

constexpr int kMqWaves = kMqThreads / 64;
constexpr int kMqChunk = 64;                        // keys per LDS chunk
constexpr int kMqChunkBytes = kMqChunk * kIdxDim * 2;
constexpr int kMqPieces = kMqChunkBytes / 16 / kMqThreads;   // 16-byte pieces per thread per chunk

__device__ __forceinline__ uint32_t mq_lds_offset(uint32_t key_local, uint32_t piece) {
  return key_local * (kIdxDim * 2) + ((piece ^ (key_local & 15u)) << 4);
}

// kQw: queries per wave (1 for query_len <= 4, 2 up to 8).
template <int kQw>
__global__ __launch_bounds__(kMqThreads) void indexer_mq_kernel(IndexerMqArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[2][kMqChunkBytes];   // 32 KiB

  const uint32_t r = row_of_block(a.blk_begin, blockIdx.x);
  const uint32_t n = a.kv_len[r];
  const uint32_t k0 = (blockIdx.x - a.blk_begin[r]) * a.keys_per_block;
  const uint32_t k_end = min(n, k0 + a.keys_per_block);
  const uint16_t *__restrict__ keys = a.keys[r];
  const uint32_t Q = a.query_len;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t col = lane & 15;
  const uint32_t grp = lane >> 4;

  const uint32_t chunks = (k_end - k0 + kMqChunk - 1) / kMqChunk;
  // Staging: piece p = tid + threads * u of a chunk is key p / 16, 16-byte
  // piece p % 16 of its row. Keys past the row's end are clamped (loaded,
  // never stored as scores).
  u32x4 st[kMqPieces];
  auto load_chunk = [&](uint32_t c) {
#pragma unroll
    for (int u = 0; u < kMqPieces; ++u) {
      const uint32_t p = tid + kMqThreads * u;
      const uint32_t key = min(k0 + kMqChunk * c + (p >> 4), n - 1);
      st[u] = load16(keys + static_cast<uint64_t>(key) * kIdxDim + 8 * (p & 15u));
    }
  };
  auto store_chunk = [&](int slot) {
#pragma unroll
    for (int u = 0; u < kMqPieces; ++u) {
      const uint32_t p = tid + kMqThreads * u;
      *reinterpret_cast<u32x4 *>(&kbuf[slot][mq_lds_offset(p >> 4, p & 15u)]) = st[u];
    }
  };
  load_chunk(0);

  // This wave's queries, their fragments (head 16m + col, features
  // [32*grp + 8c, +8)) and the head weights of the D rows of this lane.
  bf16x8 qa[kQw][4][4];
  float wt[kQw][4][4];
  bool live[kQw];
  uint32_t vis[kQw];
  float *srow[kQw];
#pragma unroll
  for (int k = 0; k < kQw; ++k) {
    const uint32_t t = wave + kMqWaves * k;
    live[k] = t < Q;
    const uint32_t tq = live[k] ? t : 0;
    const uint64_t qrow = static_cast<uint64_t>(a.q_row[r]) + tq;
    const uint16_t *q = a.q + qrow * kHeads * kIdxDim;
    const float *w = a.w + qrow * kHeads;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int c = 0; c < 4; ++c) qa[k][m][c] = as_bf16x8(load16(q + (16 * m + col) * kIdxDim + 32 * grp + 8 * c));
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[k][m][i] = w[16 * m + 4 * grp + i];
    }
    vis[k] = a.visible[r * kRowsMax + tq];
    srow[k] = a.scores + (static_cast<uint64_t>(r) * Q + tq) * a.score_stride;
  }
  store_chunk(0);
  __syncthreads();

  for (uint32_t c = 0; c < chunks; ++c) {
    const int slot = c & 1;
    load_chunk(min(c + 1, chunks - 1));   // next chunk in flight (the last is loaded again, unused)
    const unsigned char *kb = kbuf[slot];
#pragma unroll
    for (int kt = 0; kt < kMqChunk / 16; ++kt) {
      // B operand of the tile's 16 keys: key 16kt + col, pieces 4*grp + s.
      bf16x8 b[4];
      const uint32_t kl = 16 * kt + col;
#pragma unroll
      for (int s = 0; s < 4; ++s) b[s] = as_bf16x8(*reinterpret_cast<const u32x4 *>(kb + mq_lds_offset(kl, 4 * grp + s)));
      const uint32_t key = k0 + kMqChunk * c + kl;
#pragma unroll
      for (int k = 0; k < kQw; ++k) {
        if (!live[k]) continue;   // wave-uniform
        float part = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mfma16(qa[k][m][s], b[s], acc);
#pragma unroll
          for (int j = 0; j < 4; ++j) part = fmaf(fmaxf(acc[j], 0.0f), wt[k][m][j], part);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (grp == 0 && key < k_end)
          srow[k][key] = (key < vis[k] && __builtin_isfinite(part)) ? part : -__builtin_inff();
      }
    }
    // The other slot was last read in the previous iteration, before its
    // closing barrier; the barrier below publishes the next chunk.
    store_chunk(slot ^ 1);
    __syncthreads();
  }
}

hipError_t launch_indexer_mq(const IndexerMqArgs &a, uint32_t blocks, hipStream_t s) {
  if (a.query_len <= kMqWaves)
    hipLaunchKernelGGL(indexer_mq_kernel<1>, dim3(blocks), dim3(kMqThreads), 0, s, a);
  else
    hipLaunchKernelGGL(indexer_mq_kernel<2>, dim3(blocks), dim3(kMqThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
