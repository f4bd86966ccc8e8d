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
//     weights are applied in registers; after every 4 tiles two lane-row
//     swaps (v_permlane16_swap, v_permlane32_swap) finish the four head sums
//     at once, leaving lane row g with tile g's 16 scores.
//   * The workgroup stages the 16 KiB query in LDS once; each wave keeps its
//     copy of the query fragments in 64 VGPRs. Key tiles stream through a
//     ring of four register buffers, so three tiles (12 KiB) of loads are in
//     flight per wave while a fourth tile's 16 MFMAs run. A row's 16-key
//     tiles are dealt round robin over all of its waves (wave w of the row's
//     workgroup b takes tiles 4b + w, 4b + w + S, ..., S = 4 x the row's
//     workgroups), so the row's waves read neighbouring tiles at any time
//     (measured faster than a contiguous 1024-key range per workgroup; deeper
//     rings, 512-key workgroups and 8-wave workgroups measured slower).
// The arithmetic per key is a fixed instruction sequence independent of the
// row count or of other rows, so every row is bitwise identical to a
// one-row launch.
//
// Fused top-k stage (kFused, for ds_rows_indexer_topk). The pages' first
// top-k stage sorts every 1024-key block and keeps its best 512
// (deepseek_indexer_topk_block_rows_i32). Here every wave keeps, from the 256
// scores it just computed (still in its registers: after each group of 4
// tiles every lane holds one score, lane row g that of tile g), only the
// keys at or above a threshold T that keeps 3C/4 to C of them (C = 32, or 8
// when every row has at least 262144 visible keys): a search over T's bits
// with ballot counts, two bits per step and stopping at the first T in
// range, finds it without LDS or barriers. When ties at the (3C/4)-th best
// score bits T leave no such threshold, it keeps every key above T and, of
// the keys tied at T, the lowest indices (ties rank by lower index) up to C
// in all. It writes those keys and a 64-bit floor: a key no better than any
// key it did not write (T << 32 after a clean threshold; the exact key of its
// best unwritten tie otherwise). The final top-k level uses the floors to
// prove that no unkept key can reach the row's top 512, and selects from the
// scores again when one could.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"
#include "select_common.hpp"

namespace ds {

constexpr int kIdxRing = 4;   // tile buffers per wave (kIdxRing - 1 in flight)
constexpr uint32_t kIdxWaves = kIdxThreads / 64;
constexpr int kQVec = kHeads * kIdxDim / 8 / kIdxThreads;   // 16-byte query pieces per thread
// Every lane ends each group of 4 tiles with one score (lane row g: tile
// 4j + g); the fused stage queues the last four, so a wave takes at most 16
// tiles, and ring passes cover whole groups.
static_assert(kIdxRing % 4 == 0, "ring passes hold whole groups of 4 tiles");
static_assert(kIdxMaxKeysPerBlock / (kIdxThreads / 64) / kIdxTile <= 16, "tiles per wave");
static_assert((kIdxMaxKeysPerBlock / (kIdxThreads / 64) / kIdxTile + kIdxRing - 1) / kIdxRing * (kIdxRing / 4) <= 4,
              "groups of 4 tiles per wave fit the queue");

// One wave's candidates (fused stage, see above), kCand of them at most:
// o[e] are the score bits (0 = not valid) of the lane's four queued keys,
// kidx[e] their key indices. Key indices increase with (3 - e, lane): e = 3
// holds the wave's first group of tiles, and within a group lane row g holds
// tile g of the group.
template <int kCand>
__device__ __forceinline__ void wave_candidates(const IndexerArgs &a, const uint32_t (&o)[4],
                                                const uint32_t (&kidx)[4], uint32_t block, uint32_t wave,
                                                uint32_t lane) {
  constexpr uint32_t kKeep = kCand * 3 / 4;
  static_assert(kCand <= 64 && kKeep >= 1, "one slot per lane");
  constexpr uint32_t kC = kCand;
  const uint64_t slot0 = static_cast<uint64_t>(block) * (kIdxThreads / 64) * kC + wave * kC;
  const uint64_t floor_at = static_cast<uint64_t>(block) * kIdxFloors + wave;
  auto count_ge = [&](uint32_t t) -> uint32_t {   // keys of the wave with score bits >= t
    uint32_t c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) c += static_cast<uint32_t>(__popcll(__ballot(o[e] >= t)));
    return c;
  };
  const uint32_t nvalid = count_ge(1u);
  uint32_t thr = 1;   // keep every valid key
  uint32_t kept = nvalid;
  if (nvalid > kC) {
    // T is built from the top bit down, one bit per step, each time taking
    // the larger value that still has at least kKeep keys at or above it.
    // It stops as soon as the accepted T keeps at most kC keys; otherwise
    // it ends at the kKeep-th best score bits. Any T that keeps at most kC
    // keys is a valid floor: the final level's check compares the floors
    // with its 512th key, so which one is taken changes no index. If none
    // keeps at most kC, T ends as the kKeep-th best score bits (ties at T
    // overflow). The search runs on the compute unit's one scalar ALU (the
    // ballots' popcounts and sums) for every wave of the CU at once, so its
    // cost is its scalar instruction count: one count per bit takes fewer
    // in all than three counts per two bits, though the steps double.
    thr = 0;
    kept = 256;   // count_ge(0); replaced at the first accepted step (count_ge(1) = nvalid > kKeep)
    for (int b = 31; b >= 0; --b) {
      const uint32_t t1 = thr | (1u << b);
      const uint32_t n1 = count_ge(t1);
      if (n1 >= kKeep) { thr = t1; kept = n1; }
      if (kept <= kC) break;   // uniform
    }
  }
  auto prefix = [](uint64_t mask) {   // set lanes of `mask` below this lane
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
  };
  // Which queued keys this lane writes: those at or above T, or, when the
  // keys tied at T overflow the room, those above T and the first `room`
  // ties in key-index order (e = 3 .. 0, lanes ascending).
  bool take[4];
  uint64_t floor = static_cast<uint64_t>(thr) << 32;   // after a clean threshold
  if (kept <= kC) {
#pragma unroll
    for (int e = 0; e < 4; ++e) take[e] = o[e] >= thr;
    if (kept == nvalid) floor = 0;
  } else {
    uint32_t room = kC - count_ge(thr + 1);   // slots left for ties at T (> 0)
    uint32_t first_unkept = 0xFFFFFFFFu;                // index of the best unwritten tie
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      const bool tie = o[e] == thr;
      const uint64_t m = __ballot(tie);
      const uint32_t pos = prefix(m);
      take[e] = o[e] > thr || (tie && pos < room);
      const uint64_t first = __ballot(tie && pos == room);   // the first tie past the room, if in this e
      if (first != 0 && first_unkept == 0xFFFFFFFFu)
        first_unkept = __shfl(kidx[e], static_cast<int>(__builtin_ctzll(first)));
      const uint32_t n = static_cast<uint32_t>(__popcll(m));
      room = n >= room ? 0u : room - n;
    }
    kept = kC;
    floor = (static_cast<uint64_t>(thr) << 32) | static_cast<uint32_t>(~first_unkept);
  }
  uint32_t base = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint64_t mask = __ballot(take[e]);
    const uint32_t pos = base + prefix(mask);
    if (take[e]) a.cand[slot0 + pos] = (static_cast<uint64_t>(o[e]) << 32) | static_cast<uint32_t>(~kidx[e]);
    base += static_cast<uint32_t>(__popcll(mask));
  }
  if (lane >= kept && lane < kC) a.cand[slot0 + lane] = 0;   // unused slots
  if (lane == 0) a.floors[floor_at] = floor;
}

// kCand: 0 for the plain kernel (scores only), else the fused stage's
// per-wave candidate budget. kCompact (plain kernel only): a 1-D grid of one
// workgroup per block instead of the (blocks of the longest slot, slots) one.
template <int kCand, bool kCompact = false>
__global__ __launch_bounds__(kIdxThreads) void indexer_score_kernel(IndexerArgs a) {
  static_assert(!kCompact || kCand == 0, "the fused stage keeps the 2-D grid");
  constexpr bool kFused = kCand != 0;
  __shared__ u32x4 q_lds[kHeads * kIdxDim / 8];   // 16 KiB

  // 2-D grid: (workgroups of the longest slot, slots); slot r is blockIdx.y,
  // known at launch, so every argument of the slot is read in one batch of
  // scalar loads (a slot found from the block index would first wait for the
  // block table), and workgroups past the slot's own count have no keys and
  // end after the common set-up, before any store. Compact grid (the plain
  // kernel, when the 2-D grid would be mostly empty): one workgroup per block
  // of the slots' concatenated blocks, no empty ones (at workload 3, rows of
  // 1 .. 131072 keys, the 2-D grid dispatched over 1600 empty workgroups,
  // ahead of the short rows' real ones: 48.8 -> 43.5 us per step); the block
  // table and every slot's fields are loaded together and the slot is picked
  // from them with scalar compares (the compiler issues those loads in two
  // batches: about 0.5 us more per launch where the 2-D grid has few empty
  // workgroups).
  uint32_t r, blk0, blk1, n, visible, qr, srow, xb;
  uint64_t kbits;
  uint64_t qbits = reinterpret_cast<uint64_t>(a.q), wbits = reinterpret_cast<uint64_t>(a.w),
           sbits = reinterpret_cast<uint64_t>(a.scores);
  uint64_t sstride = a.score_stride;
  uint64_t tbits = reinterpret_cast<uint64_t>(a.stamps);
  if constexpr (!kCompact) {
    r = blockIdx.y;
    blk0 = a.blk_begin[r], blk1 = a.blk_begin[r + 1], n = a.kv_len[r], visible = a.visible[r];
    qr = a.q_row[r];
    kbits = reinterpret_cast<uint64_t>(a.keys[r]);
    srow = a.score_row[r];
    // One use of them all: the compiler issues these scalar loads together
    // and waits once, rather than in dependent batches ahead of their first
    // uses.
    asm volatile("" : "+s"(blk0), "+s"(blk1), "+s"(n), "+s"(visible), "+s"(qr), "+s"(kbits), "+s"(qbits),
                 "+s"(wbits), "+s"(sbits), "+s"(sstride), "+s"(tbits), "+s"(srow));
    xb = blockIdx.x;
  } else {
    uint32_t bb[kRowsMax + 1], kv[kRowsMax], vis[kRowsMax], qrs[kRowsMax], srs[kRowsMax];
    uint64_t kp[kRowsMax];
#pragma unroll
    for (int i = 0; i < kRowsMax; ++i) {
      bb[i] = a.blk_begin[i];
      kv[i] = a.kv_len[i];
      vis[i] = a.visible[i];
      qrs[i] = a.q_row[i];
      srs[i] = a.score_row[i];
      kp[i] = reinterpret_cast<uint64_t>(a.keys[i]);
    }
    bb[kRowsMax] = a.blk_begin[kRowsMax];
    static_assert(kRowsMax == 8, "the slot fields are listed one by one below");
    // (All in one statement: split, the compiler waited for the first
    // statement's loads before issuing the rest.)
    asm volatile("" : "+s"(bb[0]), "+s"(bb[1]), "+s"(bb[2]), "+s"(bb[3]), "+s"(bb[4]), "+s"(bb[5]), "+s"(bb[6]),
                 "+s"(bb[7]), "+s"(bb[8]), "+s"(kv[0]), "+s"(kv[1]), "+s"(kv[2]), "+s"(kv[3]), "+s"(kv[4]),
                 "+s"(kv[5]), "+s"(kv[6]), "+s"(kv[7]), "+s"(vis[0]), "+s"(vis[1]), "+s"(vis[2]), "+s"(vis[3]),
                 "+s"(vis[4]), "+s"(vis[5]), "+s"(vis[6]), "+s"(vis[7]), "+s"(qrs[0]), "+s"(qrs[1]), "+s"(qrs[2]),
                 "+s"(qrs[3]), "+s"(qrs[4]), "+s"(qrs[5]), "+s"(qrs[6]), "+s"(qrs[7]), "+s"(srs[0]), "+s"(srs[1]),
                 "+s"(srs[2]), "+s"(srs[3]), "+s"(srs[4]), "+s"(srs[5]), "+s"(srs[6]), "+s"(srs[7]), "+s"(kp[0]),
                 "+s"(kp[1]), "+s"(kp[2]), "+s"(kp[3]), "+s"(kp[4]), "+s"(kp[5]), "+s"(kp[6]), "+s"(kp[7]),
                 "+s"(qbits), "+s"(wbits), "+s"(sbits), "+s"(sstride), "+s"(tbits));
    const uint32_t b = blockIdx.x;
    r = 0;
#pragma unroll
    for (int i = 1; i < kRowsMax; ++i) r += b >= bb[i] ? 1u : 0u;   // slots past `rows` start at the total
    blk0 = bb[0], blk1 = bb[1], n = kv[0], visible = vis[0], qr = qrs[0], srow = srs[0], kbits = kp[0];
#pragma unroll
    for (int i = 1; i < kRowsMax; ++i) {
      if (r == static_cast<uint32_t>(i)) {
        blk0 = bb[i], blk1 = bb[i + 1], n = kv[i], visible = vis[i], qr = qrs[i], srow = srs[i], kbits = kp[i];
      }
    }
    xb = b - blk0;
  }
  // Timing stamps (ds_rows_time_next_indexer): this workgroup's start now,
  // each wave's end where it leaves.
  uint64_t *const stamps = tbits != 0 ? global_ptr<uint64_t>(tbits) +
                                            static_cast<uint64_t>(blockIdx.y * gridDim.x + blockIdx.x) * kTimerStamps
                                      : nullptr;   // (a compact grid is 1-D: blockIdx.y = 0)
  if (stamps != nullptr && threadIdx.x == 0) stamps[0] = wall_clock64();
  auto stamp_end = [&]() {
    if (stamps != nullptr && (threadIdx.x & 63) == 0) stamps[1 + (threadIdx.x >> 6)] = wall_clock64();
  };
  const uint16_t *const keys = global_ptr<const uint16_t>(kbits);
  const uint32_t nblk = blk1 - blk0;
  const bool live = xb < nblk;   // uniform (always, on a compact grid)
  // Workgroup index in the fused candidate layout: every row has room for
  // the grid's blocks per row (the widest row's), so row r's candidates and
  // floors start at block r * gridDim.x and a reader finds them from the row
  // alone (only the fused stage, which keeps the 2-D grid, uses it).
  const uint32_t block = r * gridDim.x + xb;
  // Tiles of 16 keys are dealt round robin over the row's waves: wave w of
  // the row's workgroup b takes tiles t0 = 4b + w, t0 + S, t0 + 2S, ...
  // (S = 4 x the row's workgroups), so at any time the row's waves read
  // neighbouring tiles.
  const uint32_t tstride = kIdxWaves * nblk;
  const uint16_t *__restrict__ q = global_ptr<const uint16_t>(qbits) + static_cast<uint64_t>(qr) * kHeads * kIdxDim;
  const float *__restrict__ w = global_ptr<const float>(wbits) + static_cast<uint64_t>(qr) * kHeads;
  float *__restrict__ scores = global_ptr<float>(sbits) + static_cast<uint64_t>(srow) * sstride;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t col = lane & 15;   // key within tile / head within head tile
  const uint32_t grp = lane >> 4;   // 64-byte span of the 256-byte row

  // The query and weights go out first (they gate every MFMA), then the
  // first tiles of keys; the query reaches LDS once its loads have landed.
  __shared__ float w_lds[kHeads];
  u32x4 qv[kQVec];
#pragma unroll
  for (int i = 0; i < kQVec; ++i) qv[i] = load16(q + 8 * (tid + kIdxThreads * i));
  const float wv = w[tid & (kHeads - 1)];

  const uint32_t tiles = (n + kIdxTile - 1) / kIdxTile;
  const uint32_t t0 = kIdxWaves * xb + wave;
  const uint32_t mine = live && tiles > t0 ? (tiles - t0 + tstride - 1) / tstride : 0;
  auto key_of = [&](uint32_t i) { return (t0 + tstride * i) * kIdxTile + col; };
  auto load_tile = [&](uint32_t i, u32x4 (&kb)[4]) {
    const uint32_t key = min(key_of(i), n - 1);   // tail: clamp, not stored
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
  for (int i = 0; i < kQVec; ++i) q_lds[tid + kIdxThreads * i] = qv[i];
  if (tid < kHeads) w_lds[tid] = wv;
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
  if (!live || (!kFused && mine == 0)) {   // (in the fused stage every wave of a row writes its floor)
    stamp_end();
    return;
  }

  // Tiles go in groups of 4: each lane keeps its head group's partial sum of
  // the group's tiles, then two lane-row swaps finish all four head sums at
  // once and leave lane row g with tile 4j + g (lane col: key col of it). The
  // additions are (g0 + g1) + (g2 + g3), the order of a per-tile two-step
  // cross-lane sum. Fused stage: that score is the one this lane keeps, in
  // a queue of the wave's last four groups (newest first).
  uint32_t fifo[4] = {0, 0, 0, 0};
  for (uint32_t i0 = 0; i0 < mine; i0 += kIdxRing) {
    float part[4];
#pragma unroll
    for (int u = 0; u < kIdxRing; ++u) {
      const uint32_t i = i0 + u;
      load_tile(min(i + kIdxRing - 1, last), buf[(u + kIdxRing - 1) % kIdxRing]);
      float p = 0.0f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma16(qa[m][c], as_bf16x8(buf[u][c]), acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) p = fmaf(fmaxf(acc[j], 0.0f), wt[m][j], p);
      }
      part[u & 3] = p;
      if ((u & 3) == 3) {
        const float t01 = swap_rows16_sum(part[0], part[1]);   // even rows: tile 0, odd rows: tile 1
        const float t23 = swap_rows16_sum(part[2], part[3]);   // even rows: tile 2, odd rows: tile 3
        const float sum = swap_halves_sum(t01, t23);            // lane row g: tile g of the group
        const uint32_t ti = i0 + (u - 3) + grp;
        const uint32_t key = key_of(ti);
        const float v = (key < visible && __builtin_isfinite(sum)) ? sum : -__builtin_inff();
        if (ti < mine && key < n) scores[key] = v;
        if constexpr (kFused) {
          fifo[3] = fifo[2];
          fifo[2] = fifo[1];
          fifo[1] = fifo[0];
          fifo[0] = (ti < mine && key < n) ? static_cast<uint32_t>(topk_key(v, key) >> 32) : 0u;
        }
      }
    }
  }
  if constexpr (kFused) {
    // fifo[e] holds tile i = 4 * (groups - 1 - e) + grp.
    const uint32_t groups = (mine + kIdxRing - 1) / kIdxRing * (kIdxRing / 4);
    uint32_t kidx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t i = 4 * (groups - 1 - e) + grp;   // (unused when groups <= e: fifo[e] is 0)
      kidx[e] = key_of(i);
    }
    wave_candidates<kCand>(a, fifo, kidx, block, wave, lane);
  }
  stamp_end();
}

hipError_t launch_indexer_score(const IndexerArgs &a, uint32_t max_row_blocks, uint32_t wave_cand, bool compact,
                                hipStream_t s) {
  const dim3 grid = compact ? dim3(a.blk_begin[kRowsMax]) : dim3(max_row_blocks, a.rows);
  if (compact)
    hipLaunchKernelGGL((indexer_score_kernel<0, true>), grid, dim3(kIdxThreads), 0, s, a);
  else if (wave_cand == kIdxWaveCand)
    hipLaunchKernelGGL(indexer_score_kernel<static_cast<int>(kIdxWaveCand)>, grid, dim3(kIdxThreads), 0, s, a);
  else if (wave_cand == kIdxWaveCandLong)
    hipLaunchKernelGGL(indexer_score_kernel<static_cast<int>(kIdxWaveCandLong)>, grid, dim3(kIdxThreads), 0, s, a);
  else
    hipLaunchKernelGGL(indexer_score_kernel<0>, grid, dim3(kIdxThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
