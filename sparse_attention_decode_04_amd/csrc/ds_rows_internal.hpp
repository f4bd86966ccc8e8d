// Internal interface between the C ABI (ds_rows.cpp: argument checks, tables,
// workspace layout) and the gfx950 kernels (*.hip). Each kernel takes one
// argument struct by value (it lives in the kernarg segment) and every launch
// returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "ds_rows.h"

namespace ds {

// Records the calling thread's last-error message ("ds_rows: " + the
// formatted text) and returns `st`.
ds_status record_error(ds_status st, const char *fmt, ...);

constexpr int kRowsMax = 8;
constexpr int kHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kDim = 512;
constexpr int kTopK = 512;
constexpr int kRatio = 4;
// MI355X has 8 XCDs, each with its own L2; the dispatcher hands consecutive
// workgroups of a grid to consecutive XCDs (block b -> XCD b % 8).
constexpr uint32_t kXcds = 8;
static_assert(kRowsMax <= static_cast<int>(kXcds), "one XCD per row");

// ---------------------------------------------------------------- indexer
// One workgroup of 4 waves scores `keys_per_block` consecutive keys of one
// row; waves take 16-key tiles round robin.
constexpr int kIdxThreads = 256;
constexpr int kIdxTile = 16;
constexpr uint32_t kIdxMaxKeysPerBlock = 1024;
// Fused top-k stage (ds_rows_indexer_topk): every wave of the indexer also
// writes up to C candidate keys of its own 256 keys (those at or above a
// threshold keeping 3C/4 to C of them; every valid key when it has at most C;
// when ties at its threshold T overflow, the keys above T and the
// lowest-index ties) and a 64-bit floor, a key that no unwritten key of the
// wave exceeds: 0 when it wrote every valid key, T << 32 after a clean
// threshold, else the key of its best unwritten tie. C = kIdxWaveCand, or
// kIdxWaveCandLong when every row of the call has at least kIdxLongRow
// visible keys: a row's top 512 then averages at most half a key per wave.
constexpr uint32_t kIdxWaveCand = 32;
constexpr uint32_t kIdxWaveCandLong = 8;
constexpr uint32_t kIdxLongRow = 262144;
constexpr uint32_t kIdxCand = (kIdxThreads / 64) * kIdxWaveCand;   // candidate slots per block (at most)
constexpr uint32_t kIdxFloors = kIdxThreads / 64;                   // 4 per block
constexpr uint32_t kTimerStamps = DS_TIMER_STAMPS_PER_WG;           // timing stamps per workgroup
static_assert(kTimerStamps >= 1 + kIdxThreads / 64, "a start and one end per wave");

// Per-row arrays are indexed by the grid row ("slot"): the plain kernel
// takes the rows longest first (see launch_indexer), so slot y holds row
// score_row[y]'s keys, lengths and query, and writes that row's scores.
struct IndexerArgs {
  const uint16_t *keys[kRowsMax];   // bf16 [kv_len, 128] per slot
  const uint16_t *q;                // bf16 [_, 64, 128]
  const float *w;                   // f32 [_, 64]
  float *scores;                    // f32 [rows, score_stride]
  uint64_t score_stride;
  uint32_t score_row[kRowsMax];     // the row whose scores slot y writes
  uint32_t rows;
  uint32_t keys_per_block;          // 1024 with the fused stage; the plain kernel 64 .. 1024 (a power of 2)
  uint32_t kv_len[kRowsMax];
  uint32_t visible[kRowsMax];       // min(kv_len, (start_pos + 1) / 4)
  uint32_t q_row[kRowsMax];
  uint32_t blk_begin[kRowsMax + 1]; // first block of each row; [rows..] = total
  uint64_t *cand;                   // fused: 4 C keys per block (0 = none)
  uint64_t *floors;                 // fused: kIdxFloors floors per block (one per wave)
  uint64_t *stamps;                 // timing (ds_rows_time_next_indexer) or nullptr: per workgroup of the
                                    // grid, its start and each wave's end (wall clock)
};
// Grid (max_row_blocks, a.rows): workgroup (x, y) is slot y's x-th block;
// with compact (plain kernel only), one workgroup per block, b = 0 ..
// blk_begin[kRowsMax). wave_cand: 0 for the plain kernel, else the fused
// stage's C (kIdxWaveCand or kIdxWaveCandLong).
hipError_t launch_indexer_score(const IndexerArgs &a, uint32_t max_row_blocks, uint32_t wave_cand, bool compact,
                                hipStream_t s);

// ------------------------------------------------------------------ top-k
// One selection level: every workgroup reduces a chunk of one row's
// candidates to that chunk's best 512, sorted best first. Candidates are
// 64-bit keys (order-preserving score bits << 32 | ~index); 0 = no candidate.
// The first level reads scores (chunks of 32768); later levels read the
// previous level's 512-key lists or the fused indexer's candidates: whole,
// as the final level, when every row still selecting has at most 16384 of
// them (16 per thread; 32 64-bit keys per thread would not fit the
// registers), else in chunks of 8192 keys.
constexpr int kTopkThreads = 1024;
constexpr int kTopkPerThreadFirst = 32;
constexpr int kTopkPerThreadLater = 8;
constexpr uint32_t kTopkChunkFirst = kTopkThreads * kTopkPerThreadFirst;   // 32768
constexpr uint32_t kTopkChunkLater = kTopkThreads * kTopkPerThreadLater;   // 8192
constexpr int kTopkSortCap = 1024;

struct TopkLevelArgs {
  const float *scores;              // level 0 input: f32 [rows, score_stride]
  uint64_t score_stride;
  const uint64_t *in;               // later levels: lists of the previous level
  uint64_t *out;                    // this level's lists (non-final rows)
  int32_t *indices;                 // final output
  uint32_t rows;
  uint32_t from_scores;             // 1 on the first level
  uint32_t per_thread;              // candidates per thread: 4/8/16, the smallest that holds every row's
                                    // candidates (a final level), else 32 on the first level (scores) and 8
                                    // on later ones (lists), in chunks
  uint32_t final_mask;              // bit r: this level emits row r's indices
  uint32_t count[kRowsMax];         // candidates of row r at this level
  uint64_t in_base[kRowsMax];       // element offset of row r's input in `in`
  uint64_t out_base[kRowsMax];      // element offset of row r's lists in `out`
  int32_t offset[kRowsMax];
  uint32_t out_offset[kRowsMax];
  // Final level inside the attention: the room per row of the input lists
  // (0 when they are not laid out one row per room) and of the floors.
  uint32_t list_room, floor_room;
  uint32_t blk_begin[kRowsMax + 1];
  // Candidates from the fused indexer: on the final level of a row with bit r
  // of check_mask, the result stands only if no block floor of the row says
  // that an unwritten key could rank; otherwise the row is selected again from
  // its `fallback_count` scores.
  uint32_t check_mask;
  const uint64_t *floors;
  uint32_t floor_begin[kRowsMax];
  uint32_t floor_count[kRowsMax];
  uint32_t fallback_count[kRowsMax];
};
hipError_t launch_topk_level(const TopkLevelArgs &a, uint32_t blocks, hipStream_t s);

// ----------------------------------------------------------------- gather
// One workgroup of 2 waves copies 16 slots; one wave moves one 1 KiB row per
// slot, eight slots in flight. A first small kernel clears invalid[0 .. rows),
// which the gather's workgroups then set with atomic ORs.
constexpr int kGatherThreads = 128;
constexpr int kGatherSlotsPerWave = 8;
constexpr int kGatherSlotsPerBlock = (kGatherThreads / 64) * kGatherSlotsPerWave;

struct GatherArgs {
  const uint16_t *kv[kRowsMax];     // bf16 [kv_len, 512] per row
  const int32_t *indices;
  uint16_t *gathered;               // bf16 [sum(width), 512]
  uint16_t *mask;                   // bf16 [sum(width)]
  uint32_t *invalid;                // u32 [rows]
  uint32_t rows;
  uint32_t kv_len[kRowsMax];
  uint32_t width[kRowsMax];
  uint32_t index_offset[kRowsMax];
  uint64_t slot_base[kRowsMax];     // sum of widths of the rows before r
};
// Grid (max_row_blocks, a.rows): workgroup (x, r) copies row r's slots 16x ..
// (after the clearing kernel).
hipError_t launch_gather(const GatherArgs &a, uint32_t max_row_blocks, hipStream_t s);

// -------------------------------------------------------------- attention
// Phase 1 (chunk): one workgroup of 16 waves per (row, 64-slot chunk, group
// of 16 heads) computes the logits scale * q . G for its heads, per head the chunk max
// m_c, p~ = exp(l - m_c), s_c = sum p~ and a bad flag, and the chunk's part
// of the output, O_c = p~ . G (64 heads x 512 dims, f32), on MFMA. G comes
// from the gathered operand, or (direct) from each row's KV through the
// indices. Phase 2 (combine): one workgroup per (row, 16-dim chunk) weighs
// the chunks with the sink: out = sum_c exp(m_c - m) O_c / Z.
constexpr int kAttnChunk = 64;      // slots per phase-1 workgroup
constexpr int kAttnHeadGroups = 4;  // phase-1 workgroups per chunk (16 heads each)
constexpr int kAttnDimChunk = 16;   // output dims per phase-2 workgroup

struct AttnArgs {
  const uint16_t *q;                // bf16 [_, 64, 512]
  const float *sinks;               // f32 [64]
  const uint16_t *gathered;         // bf16 [sum(width), 512] (gathered variant)
  const uint16_t *mask;             // bf16 [sum(width)] (gathered variant)
  const uint32_t *invalid;          // u32 [rows] (gathered variant): nonzero zeroes the row
  const int32_t *indices;           // i32 (direct variant)
  const uint16_t *kv[kRowsMax];     // bf16 [kv_len, 512] per row (direct variant)
  float4 *stats;                    // (m_c, s_c, bad, sink): row r at stat_base[r], [chunks][64]
  float *opart;                     // f32 O_c: row r at part_base[r], [chunks][64][512]
  float *out;                       // f32 [_, 64, 512]
  float scale;
  uint32_t rows;
  uint32_t row_chunks;              // chunks of room per row: stat_base[r] = r * row_chunks * 64, etc.
  uint32_t width[kRowsMax];
  uint32_t chunks[kRowsMax];        // ceil(width / 64)
  uint32_t q_row[kRowsMax];
  uint32_t kv_len[kRowsMax];
  uint32_t index_offset[kRowsMax];
  uint64_t slot_base[kRowsMax];
  uint64_t stat_base[kRowsMax];
  uint64_t part_base[kRowsMax];
};
// Phase-1 grid (32 * ceil(max_chunks / 8), rows): workgroup (x, r) serves
// chunk 8 (x / 32) + x % 8 of row r with head group (x / 8) % 4. Workgroups go
// to the 8 XCDs by linear id, so the four head groups of a chunk share one
// XCD (and its L2, where they read the chunk's rows). Phase-2 grid
// (512 / kAttnDimChunk, rows); its kernel takes stats, opart, out and
// row_chunks as leading (preloaded) arguments.
hipError_t launch_attn_chunks(const AttnArgs &a, bool direct, uint32_t max_chunks, hipStream_t s);
hipError_t launch_attn_combine(const AttnArgs &a, hipStream_t s);

// ------------------------------------------------ final top-k + attention
// One 1024-thread workgroup per attention chunk (blocks as the attention's
// phase 1): each runs its row's final top-k level over the fused indexer's
// candidates (t: a single final, checked level) and then its attention chunk
// on the indices it selected (a: the direct variant's arguments); rows that
// are not final at this level (clear in t.final_mask) read their indices from
// t.indices. The attention's combine kernel follows.
hipError_t launch_topk_attn(const TopkLevelArgs &t, const AttnArgs &a, uint32_t max_chunks, hipStream_t s);


// ---------------------------------------------------------- multi-query indexer
// query_len (1..8) consecutive queries per row; one workgroup of 8 waves per
// `keys_per_block` keys (a multiple of 64) of one row; wave w owns query w. Scores of query t of row r at
// (r * query_len + t) * score_stride.
constexpr int kMqMaxQueries = 8;

struct IndexerMqArgs {
  const uint16_t *keys[kRowsMax];   // bf16 [kv_len, 128] per row
  const uint16_t *q;                // bf16 [_, 64, 128]; row r's query t at q_row[r] + t
  const float *w;                   // f32 [_, 64], same rows
  float *scores;                    // f32 [rows * query_len, score_stride]
  uint64_t score_stride;
  uint32_t rows;
  uint32_t query_len;
  uint32_t keys_per_block;
  uint32_t kv_len[kRowsMax];
  uint32_t q_row[kRowsMax];
  uint32_t visible[kRowsMax * kMqMaxQueries];   // [r * 8 + t]: min(kv_len, (start_pos + t + 1) / 4)
  uint32_t blk_begin[kRowsMax + 1];
};
// Grid (max_row_blocks, a.rows): workgroup (x, r) is row r's x-th block.
hipError_t launch_indexer_mq(const IndexerMqArgs &a, uint32_t max_row_blocks, hipStream_t s);

// -------------------------------------------------------------- compressor
// One decode token of the learned KV compressor per row; one workgroup per
// row (256 threads for ratio 4, 1024 for ratio 128).
struct CompressorArgs {
  const float *kv;                  // f32 [rows, P] (P = coff * head_dim)
  const float *score;               // f32 [rows, P]
  const float *ape;                 // f32 [ratio, P]
  const float *norm;                // f32 [head_dim]
  uint16_t *out;                    // bf16 [rows, head_dim]
  float *kv_state[kRowsMax];        // f32 [coff * ratio, P] per row
  float *score_state[kRowsMax];
  uint32_t rows, ratio, head_dim;
  uint32_t start_pos[kRowsMax];
  float eps;
};
hipError_t launch_compressor(const CompressorArgs &a, hipStream_t s);

}  // namespace ds
