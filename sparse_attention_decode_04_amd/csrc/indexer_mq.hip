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
//   * Workgroup of 8 waves per `keys_per_block` keys of one row; wave w owns
//     query w (waves past query_len only help stage the keys): its 64x128
//     bf16 query fragments stay in 64 VGPRs, with the head weights of the D
//     rows each lane holds.
//   * Keys stream through LDS in chunks of 128 (32 KiB), two chunks resident
//     (one barrier per 128 keys; 64-key chunks, twice the barriers, measured
//     4% slower). A chunk is computed as two groups of four 16-key tiles.
//     Each thread's pieces of chunk c + 1 are loaded into registers while
//     chunk c is computed and stored to LDS at the end of the iteration
//     (deeper register prefetch measured no faster: the compiler then drains
//     the loads while rotating the staging registers).
//     Within a group all 64 MFMAs of the four 16-key tiles are issued before
//     the epilogues read their results. In LDS the sixteen 16-byte
//     pieces of key row k are permuted (piece j at slot j ^ (k mod 16)), so
//     the MFMA operand reads of 16 consecutive keys hit 16 different slots.
//   * MFMA 16x16x32 with M = 16 heads, N = 16 keys, K = 32 features: lane l
//     takes key l%16 and the 64-byte span [64*(l/16), +64) of its row, step c
//     the 16 bytes at 16c of it; the query fragments use the same feature
//     assignment. ReLU and head weights are applied in registers; after a
//     group's four tiles, two lane-row swaps (v_permlane16_swap,
//     v_permlane32_swap) finish the head sums of all four at once, leaving
//     lane l with key l of the group, so the scores go out as one 256-byte
//     store per wave. The additions keep the single-query indexer's order,
//     so query_len = 1 gives its bits.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

constexpr int kMqChunk = 128;                       // keys per LDS chunk (one barrier per chunk)
constexpr int kMqGroups = kMqChunk / 64;            // 64-key groups of four 16-key tiles per chunk
constexpr int kMqChunkBytes = kMqChunk * kIdxDim * 2;
constexpr int kMqDepth = 1;                         // chunks in flight ahead of the one computed

__device__ __forceinline__ uint32_t mq_lds_offset(uint32_t key_local, uint32_t piece) {
  return key_local * (kIdxDim * 2) + ((piece ^ (key_local & 15u)) << 4);
}

// kWaves waves per workgroup; wave w owns query w (waves past query_len only
// stage keys).
template <int kWaves>
__global__ __launch_bounds__(64 * kWaves) void indexer_mq_kernel(IndexerMqArgs a) {
  constexpr int kThreads = 64 * kWaves;
  constexpr int kPieces = kMqChunkBytes / 16 / kThreads;   // 16-byte pieces per thread per chunk
  constexpr int kTiles = 4;   // 16-key tiles per group
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[2][kMqChunkBytes];   // 32 KiB

  // Grid: (workgroups of the longest row, rows); row r is blockIdx.y, so the
  // row's arguments are read in one batch of scalar loads, waited for once
  // (see the single-query indexer). Workgroups past the row's own count end.
  const uint32_t r = blockIdx.y;
  uint32_t blk0 = a.blk_begin[r], blk1 = a.blk_begin[r + 1], n = a.kv_len[r], kpb = a.keys_per_block;
  uint32_t Q = a.query_len, q_row = a.q_row[r];
  uint64_t kbits = reinterpret_cast<uint64_t>(a.keys[r]), qbits = reinterpret_cast<uint64_t>(a.q),
           wbits = reinterpret_cast<uint64_t>(a.w), sbits = reinterpret_cast<uint64_t>(a.scores);
  uint64_t sstride = a.score_stride;
  asm volatile("" : "+s"(blk0), "+s"(blk1), "+s"(n), "+s"(kpb), "+s"(Q), "+s"(q_row), "+s"(kbits), "+s"(qbits),
               "+s"(wbits), "+s"(sbits), "+s"(sstride));
  if (blockIdx.x >= blk1 - blk0) return;   // uniform
  const uint32_t k0 = blockIdx.x * kpb;
  const uint32_t k_end = min(n, k0 + kpb);
  const uint16_t *__restrict__ keys = global_ptr<const uint16_t>(kbits);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t col = lane & 15;
  const uint32_t grp = lane >> 4;

  const uint32_t chunks = (k_end - k0 + kMqChunk - 1) / kMqChunk;
  // Staging: piece p = tid + threads * u of a chunk is key p / 16, 16-byte
  // piece p % 16 of its row. Keys past the row's end are clamped (loaded,
  // never stored as scores).
  // Chunk c's pieces sit in staging set c % kMqDepth from their load, issued
  // kMqDepth chunks ahead, until they are stored to LDS slot c % 2 at the end
  // of the iteration before c (kMqDepth = 1: one set, one chunk ahead).
  u32x4 st[kMqDepth][kPieces];
  auto load_chunk = [&](uint32_t c, u32x4 (&set)[kPieces]) {
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const uint32_t p = tid + kThreads * u;
      const uint32_t key = min(k0 + kMqChunk * c + (p >> 4), n - 1);
      set[u] = load16(keys + static_cast<uint64_t>(key) * kIdxDim + 8 * (p & 15u));
    }
  };
  auto store_chunk = [&](int slot, const u32x4 (&set)[kPieces]) {
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
      const uint32_t p = tid + kThreads * u;
      *reinterpret_cast<u32x4 *>(&kbuf[slot][mq_lds_offset(p >> 4, p & 15u)]) = set[u];
    }
  };
#pragma unroll
  for (int d = 0; d < kMqDepth; ++d) load_chunk(min(static_cast<uint32_t>(d), chunks - 1), st[d]);

  // This wave's query: its fragments (head 16m + col, features
  // [32*grp + 8s, +8)) and the head weights of the D rows of this lane.
  const bool live = wave < Q;   // wave-uniform
  const uint32_t t = live ? wave : 0;
  const uint64_t qrow = static_cast<uint64_t>(q_row) + t;
  bf16x8 qa[4][4];
  float wt[4][4];
  {
    const uint16_t *q = global_ptr<const uint16_t>(qbits) + qrow * kHeads * kIdxDim;
    const float *w = global_ptr<const float>(wbits) + qrow * kHeads;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int s = 0; s < 4; ++s) qa[m][s] = as_bf16x8(load16(q + (16 * m + col) * kIdxDim + 32 * grp + 8 * s));
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[m][i] = w[16 * m + 4 * grp + i];
    }
  }
  const uint32_t vis = a.visible[r * kRowsMax + t];
  float *srow = global_ptr<float>(sbits) + (static_cast<uint64_t>(r) * Q + t) * sstride;
  // Every load issued so far (the query, weights and first chunks) has
  // landed: without this wait the compiler, unsure whether the query's
  // loads are done when the loop starts, would wait for the in-flight
  // chunks inside every iteration.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  store_chunk(0, st[0]);
  __syncthreads();

  const float inf = opaque_inf();   // for relu_num
  for (uint32_t c0 = 0; c0 < chunks; c0 += kMqDepth) {
#pragma unroll
   for (int u = 0; u < kMqDepth; ++u) {
    const uint32_t c = c0 + u;
    if (c >= chunks) break;   // uniform
    const int slot = c & 1;
    // Set u (chunk c) is in LDS already: refill it with chunk c + depth
    // (past the end, the last chunk again, unused).
    load_chunk(min(c + kMqDepth, chunks - 1), st[u]);
    if (live) {
      const unsigned char *kb = kbuf[slot];
      // Tile kt: B operand (key 16kt + col, pieces 4*grp + s), read one tile
      // ahead of its products; the four head tiles' accumulators are issued
      // step by step so that their chains interleave.
      for (int g = 0; g < kMqGroups; ++g) {
      auto read_b = [&](int kt, bf16x8 (&b)[4]) {
        const uint32_t kl = 64 * g + 16 * kt + col;
#pragma unroll
        for (int s = 0; s < 4; ++s) b[s] = as_bf16x8(*reinterpret_cast<const u32x4 *>(kb + mq_lds_offset(kl, 4 * grp + s)));
      };
      auto products = [&](const bf16x8 (&b)[4], f32x4 (&acc)[4]) {
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int m = 0; m < 4; ++m) acc[m] = mfma16(qa[m][s], b[s], acc[m]);
        }
      };
      // part[kt]: this lane's head-group sum for key 16kt + col.
      auto epilogue = [&](const f32x4 (&acc)[4]) {
        float part = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int j = 0; j < 4; ++j) part = fmaf(relu_num(acc[m][j], inf), wt[m][j], part);
        }
        return part;
      };
      // All four tiles' products first (B read one tile ahead), then the
      // epilogues: every MFMA result is long complete when it is read.
      bf16x8 b0[4], b1[4];
      f32x4 acc[kTiles][4];
      float part[kTiles];
      read_b(0, b0);
      read_b(1, b1);
      __builtin_amdgcn_s_setprio(1);
      products(b0, acc[0]);
      read_b(2, b0);
      products(b1, acc[1]);
      read_b(3, b1);
      products(b0, acc[2]);
      products(b1, acc[3]);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int kt = 0; kt < kTiles; ++kt) part[kt] = epilogue(acc[kt]);
      // Head sums of the chunk's four tiles at once: lane row g (16 lanes)
      // holds the partial of head group g for every tile; two swaps of lane
      // rows leave lane row g with the full sum of tile g, added in the order
      // (g0 + g1) + (g2 + g3) of the single-query indexer. Lane l then holds
      // key 64c + l of the chunk.
      const float t01 = swap_rows16_sum(part[0], part[1]);   // even rows: tile 0, odd rows: tile 1
      const float t23 = swap_rows16_sum(part[2], part[3]);   // even rows: tile 2, odd rows: tile 3
      const float sum = swap_halves_sum(t01, t23);            // lane row g: tile g
      const uint32_t key = k0 + kMqChunk * c + 64 * g + lane;
      if (key < k_end) srow[key] = (key < vis && __builtin_isfinite(sum)) ? sum : -__builtin_inff();
      }
    }
    // The other slot was last read in the previous iteration, before its
    // closing barrier; the barrier below publishes the next chunk.
    store_chunk(slot ^ 1, st[(u + 1) % kMqDepth]);
    __syncthreads();
   }
  }
}

hipError_t launch_indexer_mq(const IndexerMqArgs &a, uint32_t max_row_blocks, hipStream_t s) {
  hipLaunchKernelGGL(indexer_mq_kernel<kMqMaxQueries>, dim3(max_row_blocks, a.rows), dim3(64 * kMqMaxQueries), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
