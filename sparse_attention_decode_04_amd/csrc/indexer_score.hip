// Lightning-indexer score of one query per row, bf16 MFMA on gfx950.
//
// Computes, for key j of row r,
//   s[j] = sum_h w[h] * max(0, sum_d q[h,d] * k[j,d])      (64 heads, d < 128)
// and stores -inf for keys at or past the causal limit or with a non-finite
// score. Source: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernel deepseek_indexer_score_mma_rows_bf16 (score, ReLU, head-weight
// epilogue, causal mask, finite check).
//
// Mapping (differs from the pages' Metal design: no staging of keys, no fp16
// conversion; bf16 products are exact in the f32 accumulator):
//   * MFMA 16x16x32 with M = 16 heads, N = 16 keys, K = 32 features; four
//     head tiles x four feature steps per 16-key tile.
//   * Lane l of a wave serves key l%16 and the 64 contiguous bytes
//     [64*(l/16), +64) of that key's 256-byte row: feature step c uses bytes
//     16c of that span. The query fragments use the same feature assignment,
//     so the contraction is unchanged and no key data is shuffled.
//   * D lane l holds heads 16m + 4*(l/16) + i of key l%16: the ReLU and head
//     weights are applied in registers, then two cross-lane adds finish the
//     head sum.
//   * The workgroup stages the 16 KiB query in LDS once; each wave keeps its
//     copy of the query fragments in 64 VGPRs. Key tiles stream through a
//     ring of four register buffers, so three tiles (12 KiB) of loads are in
//     flight per wave while a fourth tile's 16 MFMAs run.
// The arithmetic per key is a fixed instruction sequence independent of the
// row count or of other rows, so every row is bitwise identical to a
// one-row launch.
//
// Fused top-k stage (kFused, for ds_rows_indexer_topk). The pages' first
// top-k stage sorts every 1024-key block and keeps its best 512
// (deepseek_indexer_topk_block_rows_i32); here the workgroup, with its
// block's scores still in LDS, keeps only the keys of its top score bins: at
// least 64 of them (or all valid keys when there are at most 128), at most
// 128. Linear bins over the block's own score range are monotone in the score,
// so every key it does not keep ranks below every key it keeps; it writes the
// smallest kept key as the block's floor. The final top-k level uses the
// floors to prove that no unkept key can reach the row's top 512.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"
#include "select_common.hpp"

namespace ds {

constexpr int kIdxRing = 4;   // tile buffers per wave (kIdxRing - 1 in flight)

// The block's candidates (fused stage, see above): scores of its keys as
// order-preserving bits (0 = not valid) in LDS, 4 per thread.
__device__ __forceinline__ void block_candidates(const IndexerArgs &a, const uint32_t *s_ord, uint32_t *s_hist,
                                                 uint32_t *s_misc, unsigned long long *s_floor, uint32_t k0) {
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  constexpr int kPer = kIdxMaxKeysPerBlock / kIdxThreads;   // 4
  uint32_t o[kPer];
  uint32_t nvalid = 0, omin1 = 0xFFFFFFFFu, omax = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    o[j] = s_ord[tid + kIdxThreads * j];
    nvalid += o[j] != 0 ? 1u : 0u;
    omin1 = min(omin1, o[j] - 1u);   // a missing key (0) wraps to the maximum
    omax = max(omax, o[j]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    nvalid += static_cast<uint32_t>(__shfl_xor(static_cast<int>(nvalid), off));
    omin1 = min(omin1, static_cast<uint32_t>(__shfl_xor(static_cast<int>(omin1), off)));
    omax = max(omax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(omax), off)));
  }
  if (lane == 0) {
    atomicAdd(&s_misc[0], nvalid);
    atomicMin(&s_misc[1], omin1);
    atomicMax(&s_misc[2], omax);
  }
  __syncthreads();
  const uint32_t total = s_misc[0];
  const float smin = ord_score(s_misc[1] + 1u), smax = ord_score(s_misc[2]);
  const float range = smax - smin;
  const float scale = (range > 0.0f && __builtin_isfinite(range)) ? static_cast<float>(kIdxCandBins) / range : 0.0f;
  uint32_t bin[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const float x = (ord_score(o[j]) - smin) * scale;
    bin[j] = o[j] != 0 ? static_cast<uint32_t>(fminf(x, static_cast<float>(kIdxCandBins - 1)))
                       : static_cast<uint32_t>(kIdxCandBins);
  }
  // Lowest kept bin: every bin when the block has at most kIdxCand valid
  // keys, otherwise the highest bin at which kIdxCandMin keys lie at or above.
  uint32_t lo = 0, kept = total;
  if (total > kIdxCand) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) hist_add(s_hist, bin[j], kIdxCandBins, lane);
    __syncthreads();
    if (tid < 64) {   // wave 0: lane l scans bins 255 - 4l .. 252 - 4l
      uint32_t v[4], sum = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) { v[k] = s_hist[kIdxCandBins - 1 - 4 * tid - k]; sum += v[k]; }
      uint32_t incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t up = __shfl_up(incl, off);
        if (tid >= static_cast<uint32_t>(off)) incl += up;
      }
      uint32_t before = incl - sum;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (before < kIdxCandMin && kIdxCandMin <= before + v[k]) {
          s_misc[3] = kIdxCandBins - 1 - 4 * tid - k;
          s_misc[4] = before + v[k];
        }
        before += v[k];
      }
    }
    __syncthreads();
    lo = s_misc[3];
    kept = s_misc[4];
  }
  const uint64_t blk = blockIdx.x;
  uint64_t *cand = a.cand + blk * kIdxCand;
  if (kept > kIdxCand) {
    // Heavy ties in the boundary bin: write nothing; the floor ~0 makes the
    // row fall back to a selection over its scores.
    if (tid < kIdxCand) cand[tid] = 0;
    if (tid == 0) a.floors[blk] = ~0ull;
    return;
  }
  uint64_t mine = ~0ull;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (bin[j] < static_cast<uint32_t>(kIdxCandBins) && bin[j] >= lo) {
      const uint32_t key_index = k0 + tid + kIdxThreads * j;
      const uint64_t kk = (static_cast<uint64_t>(o[j]) << 32) | static_cast<uint32_t>(~key_index);
      cand[atomicAdd(&s_misc[5], 1u)] = kk;
      mine = min(mine, kk);
    }
  }
  if (tid >= kept && tid < kIdxCand) cand[tid] = 0;   // unused slots
  // The floor: the smallest kept key, or 0 when every valid key was kept.
  uint64_t m = mine;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t ohi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(m >> 32)), off));
    const uint32_t olo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(m)), off));
    m = min(m, (static_cast<uint64_t>(ohi) << 32) | olo);
  }
  if (lane == 0) atomicMin(s_floor, static_cast<unsigned long long>(m));
  __syncthreads();
  if (tid == 0) a.floors[blk] = kept == total ? 0ull : static_cast<uint64_t>(*s_floor);
}

template <bool kFused>
__global__ __launch_bounds__(kIdxThreads) void indexer_score_kernel(IndexerArgs a) {
  __shared__ u32x4 q_lds[kHeads * kIdxDim / 8];   // 16 KiB
  __shared__ uint32_t s_ord[kFused ? kIdxMaxKeysPerBlock : 1];
  __shared__ uint32_t s_hist[kFused ? kIdxCandBins : 1];
  __shared__ uint32_t s_misc[8];
  __shared__ unsigned long long s_floor;

  const uint32_t r = row_of_block(a.blk_begin, blockIdx.x);
  const uint32_t n = a.kv_len[r];
  const uint32_t visible = a.visible[r];
  const uint32_t k0 = (blockIdx.x - a.blk_begin[r]) * a.keys_per_block;
  const uint32_t k_end = min(n, k0 + a.keys_per_block);
  const uint16_t *__restrict__ keys = a.keys[r];
  const uint16_t *__restrict__ q = a.q + static_cast<uint64_t>(a.q_row[r]) * kHeads * kIdxDim;
  const float *__restrict__ w = a.w + static_cast<uint64_t>(a.q_row[r]) * kHeads;
  float *__restrict__ scores = a.scores + static_cast<uint64_t>(r) * a.score_stride;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t col = lane & 15;   // key within tile / head within head tile
  const uint32_t grp = lane >> 4;   // 64-byte span of the 256-byte row

  // The query and weights go out first (they gate every MFMA), then the
  // first tiles of keys; the query reaches LDS once its loads have landed.
  __shared__ float w_lds[kHeads];
  u32x4 qv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qv[i] = load16(q + 8 * (tid + kIdxThreads * i));
  const float wv = w[tid & (kHeads - 1)];

  const uint32_t tiles = (k_end - k0 + kIdxTile - 1) / kIdxTile;
  const uint32_t mine = tiles > wave ? (tiles - wave + 3) / 4 : 0;   // tiles wave, wave+4, ...
  auto load_tile = [&](uint32_t i, u32x4 (&kb)[4]) {
    const uint32_t key = min(k0 + (wave + 4 * i) * kIdxTile + col, n - 1);   // tail: clamp, not stored
    const uint16_t *krow = keys + static_cast<uint64_t>(key) * kIdxDim + 32 * grp;
#pragma unroll
    for (int c = 0; c < 4; ++c) kb[c] = load16(krow + 8 * c);
  };
  // Loads are never conditional: a tile index past the wave's last tile is
  // clamped to it (the extra tile is computed and dropped). Conditional loads
  // would make the compiler wait for every outstanding load before each
  // tile's MFMAs instead of keeping kIdxRing - 1 tiles in flight.
  u32x4 buf[kIdxRing][4];
  const uint32_t last = mine > 0 ? mine - 1 : 0;
#pragma unroll
  for (int p = 0; p < kIdxRing - 1; ++p) load_tile(min(static_cast<uint32_t>(p), last), buf[p]);
#pragma unroll
  for (int i = 0; i < 4; ++i) q_lds[tid + kIdxThreads * i] = qv[i];
  if (tid < kHeads) w_lds[tid] = wv;
  if constexpr (kFused) {
#pragma unroll
    for (int j = 0; j < static_cast<int>(kIdxMaxKeysPerBlock / kIdxThreads); ++j) s_ord[tid + kIdxThreads * j] = 0;
    s_hist[tid] = 0;
    if (tid == 0) {
      s_misc[0] = 0; s_misc[1] = 0xFFFFFFFFu; s_misc[2] = 0; s_misc[3] = 0; s_misc[4] = 0; s_misc[5] = 0;
      s_floor = ~0ull;
    }
  }
  __syncthreads();
  // Query fragments (head 16m + col, features [32*grp + 8c, +8)) and the head
  // weights of the D rows this lane holds.
  bf16x8 qa[4][4];
  float wt[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int c = 0; c < 4; ++c) qa[m][c] = as_bf16x8(q_lds[((16 * m + col) * kIdxDim + 32 * grp + 8 * c) / 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i) wt[m][i] = w_lds[16 * m + 4 * grp + i];
  }
  if (!kFused && mine == 0) return;   // (the fused stage below needs every wave)

  for (uint32_t i0 = 0; i0 < mine; i0 += kIdxRing) {
#pragma unroll
    for (int u = 0; u < kIdxRing; ++u) {
      const uint32_t i = i0 + u;
      load_tile(min(i + kIdxRing - 1, last), buf[(u + kIdxRing - 1) % kIdxRing]);
      float part = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma16(qa[m][c], as_bf16x8(buf[u][c]), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) part = fmaf(fmaxf(acc[j], 0.0f), wt[m][j], part);
      }
      // Sum the four 16-head groups held by lanes col, col+16, col+32, col+48.
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      const uint32_t key = k0 + (wave + 4 * i) * kIdxTile + col;
      if (i < mine && grp == 0 && key < k_end) {
        const float v = (key < visible && __builtin_isfinite(part)) ? part : -__builtin_inff();
        scores[key] = v;
        if constexpr (kFused) s_ord[key - k0] = static_cast<uint32_t>(topk_key(v, key) >> 32);
      }
    }
  }
  if constexpr (kFused) {
    __syncthreads();
    block_candidates(a, s_ord, s_hist, s_misc, &s_floor, k0);
  }
}

hipError_t launch_indexer_score(const IndexerArgs &a, uint32_t blocks, bool fused, hipStream_t s) {
  if (fused)
    hipLaunchKernelGGL(indexer_score_kernel<true>, dim3(blocks), dim3(kIdxThreads), 0, s, a);
  else
    hipLaunchKernelGGL(indexer_score_kernel<false>, dim3(blocks), dim3(kIdxThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
