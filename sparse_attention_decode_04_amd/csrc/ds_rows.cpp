// C ABI of the multi-row sparse-attention decode core: argument checks,
// per-row tables, workspace layout and kernel launches.
//
// The checks cover what the host dispatch code on docs.rs "mlx-native 0.21.0
// src/ops/deepseek_rows.rs" requires of its rows dispatches (row count,
// per-row lengths and positions, the causal length, the index range, disjoint
// outputs, unique query rows, buffer capacities), organised here as one pass
// over each table's fields followed by the cross-row checks (sorted ranges,
// distinct query rows). Every check runs before anything is enqueued, so a
// failed call has no effect on the device.
#include "ds_rows.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>

#include "ds_rows_internal.hpp"

namespace {

thread_local std::string g_error;

ds_status fail(const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = std::string("ds_rows: ") + buf;
  return DS_ERR_INVALID_ARGUMENT;
}

ds_status hip_fail(hipError_t e, const char *what) {
  g_error = std::string("ds_rows: ") + what + ": " + hipGetErrorString(e);
  return DS_ERR_HIP;
}

// The current device must be a gfx950 (the only target the kernels are built
// for). The answer is cached per device id; hipGetDevice itself is cheap.
ds_status check_device() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    g_error = std::string("ds_rows: no current HIP device (") + hipGetErrorString(e) + ")";
    return DS_ERR_DEVICE;
  }
  constexpr int kMaxDevices = 64;
  static std::atomic<int> verdict[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
  int v = dev < kMaxDevices ? verdict[dev].load(std::memory_order_relaxed) : 0;
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_error = "ds_rows: cannot read the properties of HIP device " + std::to_string(dev);
      return DS_ERR_DEVICE;
    }
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (v == 2) g_error = std::string("ds_rows: HIP device ") + std::to_string(dev) + " is " + prop.gcnArchName +
                          "; the kernels are built for gfx950 only";
    if (dev < kMaxDevices) verdict[dev].store(v, std::memory_order_relaxed);
  } else if (v == 2) {
    g_error = "ds_rows: HIP device " + std::to_string(dev) + " is not a gfx950; the kernels are built for it only";
  }
  return v == 1 ? DS_OK : DS_ERR_DEVICE;
}

uint32_t div_up(uint64_t a, uint64_t b) { return static_cast<uint32_t>((a + b - 1) / b); }
uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

ds_status check_row_count(uint32_t rows) {
  if (rows < 1 || rows > DS_ROWS_MAX) return fail("row table has rows = %u; a call takes 1 to %d rows", rows, DS_ROWS_MAX);
  return DS_OK;
}

// Table rows a and b whose [start, start + len) ranges intersect, if any:
// sort the starts, then compare neighbours.
bool overlapping_pair(const uint64_t *start, uint64_t len, uint32_t n, uint32_t *a, uint32_t *b) {
  std::pair<uint64_t, uint32_t> s[DS_ROWS_MAX];
  for (uint32_t i = 0; i < n; ++i) s[i] = {start[i], i};
  std::sort(s, s + n);
  for (uint32_t i = 1; i < n; ++i)
    if (s[i].first < s[i - 1].first + len) {
      *a = std::min(s[i - 1].second, s[i].second);
      *b = std::max(s[i - 1].second, s[i].second);
      return true;
    }
  return false;
}

// ------------------------------------------------------------ indexer table
struct IndexerPlan {
  uint32_t rows = 0;
  uint64_t max_kv = 0;
  uint32_t visible[ds::kRowsMax] = {};
  uint64_t q_rows = 0;          // max q_row + 1
  uint64_t indices_end = 0;     // max output_offset + 512
  uint64_t topk_bank = 0;       // u64 entries per ping-pong bank
  // Indexer grid: blocks of kIndexerKeysPerBlock keys, rows in order.
  uint32_t blk_begin[ds::kRowsMax + 1] = {};
  // Fused indexer + top-k: candidate lists, block floors, list banks.
  uint64_t fused_bank = 0;
};

constexpr uint32_t kIndexerKeysPerBlock = 1024;
// The plain score kernel (no fused stage) takes smaller blocks when a call has
// few keys: the largest power of two from 1024 down to 64 keys that gives the
// call at least one workgroup per compute unit. A workgroup streams its keys
// at a rate set by its own loads in flight, so a call with fewer, longer
// blocks than compute units (one 1024-key row, or a few long rows among short
// ones) leaves most of the GPU idle.
constexpr uint32_t kPlainMinKeysPerBlock = 64;
constexpr uint64_t kPlainMinBlocks = 256;
uint32_t plain_keys_per_block(const ds_indexer_rows *rows, uint32_t nrows) {
  uint32_t kpb = kIndexerKeysPerBlock;
  for (; kpb > kPlainMinKeysPerBlock; kpb /= 2) {
    uint64_t blocks = 0;
    for (uint32_t r = 0; r < nrows; ++r) blocks += div_up(rows->kv_len[r], kpb);
    if (blocks >= kPlainMinBlocks) break;
  }
  return kpb;
}

// One indexer row's fields: length, position, causal length and index range.
// Returns the keys visible to the row's query in *visible.
ds_status check_indexer_row(uint32_t r, uint32_t kv_len, uint32_t start_pos, int32_t offset, uint32_t *visible) {
  if (kv_len == 0) return fail("indexer row %u: kv_len is 0; every row needs at least one key", r);
  if (kv_len > DS_KV_LEN_MAX)
    return fail("indexer row %u: kv_len %u is above DS_KV_LEN_MAX = 2^30 - 1", r, kv_len);
  if (start_pos == UINT32_MAX)
    return fail("indexer row %u: start_pos 4294967295 has no next position; it must be at most 2^32 - 2", r);
  const uint32_t causal = (start_pos + 1) / DS_RATIO;
  if (causal > kv_len)
    return fail("indexer row %u: start_pos %u makes %u keys visible but kv_len is only %u", r, start_pos, causal,
                kv_len);
  if (offset < 0) return fail("indexer row %u: offset %d is negative (index -1 marks an empty slot)", r, offset);
  if (causal > 0 && int64_t(offset) + int64_t(causal) - 1 > int64_t(INT32_MAX))
    return fail("indexer row %u: the largest emitted index, offset %d + %u - 1, does not fit in int32", r, offset,
                causal);
  *visible = causal;
  return DS_OK;
}

// Scores per thread of a selection level over scores whose rows hold up to
// max_count of them: 4, 8 or 16 when every row fits one chunk (the final
// level); else chunks of 16384 (16 per thread: twice the workgroups at half
// the work of 32768) as long as every row's lists then still fit one final
// level of 4 per thread (at most 8 chunks), else chunks of 32768.
uint32_t scores_per_thread(uint32_t max_count) {
  for (uint32_t per : {4u, 8u, 16u})
    if (max_count <= ds::kTopkThreads * per) return per;
  return max_count <= 8u * ds::kTopkThreads * 16 ? 16u : static_cast<uint32_t>(ds::kTopkPerThreadFirst);
}

ds_status check_indexer(const ds_indexer_rows *t, IndexerPlan *p) {
  if (!t) return fail("indexer row table is null");
  if (const ds_status st = check_row_count(t->rows)) return st;
  p->rows = t->rows;
  for (uint32_t r = 0; r < t->rows; ++r) {
    if (const ds_status st = check_indexer_row(r, t->kv_len[r], t->start_pos[r], t->offset[r], &p->visible[r]))
      return st;
    p->max_kv = std::max<uint64_t>(p->max_kv, t->kv_len[r]);
    p->q_rows = std::max<uint64_t>(p->q_rows, uint64_t(t->q_row[r]) + 1);
    p->indices_end = std::max<uint64_t>(p->indices_end, uint64_t(t->output_offset[r]) + DS_TOP_K);
    const uint32_t blocks = div_up(t->kv_len[r], kIndexerKeysPerBlock);
    p->blk_begin[r + 1] = p->blk_begin[r] + blocks;
    const uint32_t fchunks = div_up(uint64_t(blocks) * ds::kIdxCand, ds::kTopkChunkLater);
    if (fchunks > 1) p->fused_bank += uint64_t(fchunks) * DS_TOP_K;
  }
  for (uint32_t r = t->rows; r < ds::kRowsMax; ++r) p->blk_begin[r + 1] = p->blk_begin[r];
  // The list banks of a selection from the scores: the first level's chunks
  // of every row it splits (later levels write fewer lists).
  uint32_t max_visible = 0;
  for (uint32_t r = 0; r < t->rows; ++r) max_visible = std::max(max_visible, p->visible[r]);
  const uint64_t first_chunk = uint64_t(ds::kTopkThreads) * scores_per_thread(max_visible);
  for (uint32_t r = 0; r < t->rows; ++r) {
    const uint32_t chunks = std::max<uint32_t>(1, div_up(p->visible[r], first_chunk));
    if (chunks > 1) p->topk_bank += uint64_t(chunks) * DS_TOP_K;
  }
  uint64_t starts[DS_ROWS_MAX];
  for (uint32_t r = 0; r < t->rows; ++r) starts[r] = t->output_offset[r];
  uint32_t a, b;
  if (overlapping_pair(starts, DS_TOP_K, t->rows, &a, &b))
    return fail("indexer rows %u and %u: their 512-index output ranges at %u and %u intersect", a, b,
                t->output_offset[a], t->output_offset[b]);
  return DS_OK;
}

uint64_t topk_workspace_bytes(const IndexerPlan &p) { return 2 * p.topk_bank * sizeof(uint64_t); }

// Fused workspace: candidate lists (kIdxCand keys per indexer block), wave
// floors (kIdxFloors per block), then two ping-pong banks of list keys. Every
// row has room for the widest row's blocks (the fused indexer's grid width),
// so row r's candidates and floors start at block r * room.
uint32_t fused_room_blocks(const IndexerPlan &p) {
  uint32_t room = 1;
  for (uint32_t r = 0; r < p.rows; ++r) room = std::max(room, p.blk_begin[r + 1] - p.blk_begin[r]);
  return room;
}
uint64_t fused_cand_bytes(const IndexerPlan &p) {
  return align256(uint64_t(p.rows) * fused_room_blocks(p) * ds::kIdxCand * sizeof(uint64_t));
}
uint64_t fused_floor_bytes(const IndexerPlan &p) {
  return align256(uint64_t(p.rows) * fused_room_blocks(p) * ds::kIdxFloors * sizeof(uint64_t));
}
uint64_t fused_workspace_bytes(const IndexerPlan &p) {
  return fused_cand_bytes(p) + fused_floor_bytes(p) + 2 * p.fused_bank * sizeof(uint64_t);
}

// ds_rows_indexer_topk keeps the first selection stage in the indexer only
// when every row has at least this many visible keys. Each wave keeps about
// 24 of its 256 keys, so a row's candidates can hold its top 512 only past
// ~5.5K keys, and below ~16K a wave often holds more than 24 of them (the
// row then falls back to a selection over its scores): such calls run the
// separate score and top-k kernels instead, which give the same result.
constexpr uint32_t kFusedMinVisible = 16384;

bool fused_rows(const IndexerPlan &p) {
  for (uint32_t r = 0; r < p.rows; ++r)
    if (p.visible[r] < kFusedMinVisible) return false;
  return true;
}

// The fused stage's candidates per wave: 8 (of 256 keys, keeping 6 to 8)
// when every row has at least 262144 visible keys, else 32 (keeping 24 to
// 32). A wave holds on average 512 * 256 / visible of its row's top 512, at
// most 0.5 past 262144 keys; that more than 6 of them fall in one wave (which
// sends the row to the reselection from scores) then has a chance of about
// 1e-3 per row at 262144 keys and under 1e-6 at 1M. The smaller budget
// leaves a row of up to 512K keys at most 16384 candidates, which the final
// selection takes at once.
uint32_t fused_wave_cand(const IndexerPlan &p) {
  for (uint32_t r = 0; r < p.rows; ++r)
    if (p.visible[r] < ds::kIdxLongRow) return ds::kIdxWaveCand;
  return ds::kIdxWaveCandLong;
}


// Enough for either path (and for ds_rows_indexer_candidates).
uint64_t indexer_topk_workspace_bytes(const IndexerPlan &p) {
  return std::max(fused_workspace_bytes(p), topk_workspace_bytes(p));
}

// ------------------------------------------------------------- sparse table
struct SparsePlan {
  uint32_t rows = 0;
  uint64_t q_rows = 0;
  uint64_t index_end = 0;
  uint64_t slots = 0;                  // sum of widths
  uint64_t slot_base[ds::kRowsMax] = {};
  uint32_t chunks[ds::kRowsMax] = {};
  uint64_t stat_base[ds::kRowsMax] = {};
  uint64_t part_base[ds::kRowsMax] = {};
  uint64_t stat_elems = 0, part_elems = 0;
  uint32_t max_chunks = 0;
};

ds_status check_sparse(const ds_sparse_rows *t, SparsePlan *p) {
  if (!t) return fail("sparse row table is null");
  if (const ds_status st = check_row_count(t->rows)) return st;
  p->rows = t->rows;
  for (uint32_t r = 0; r < t->rows; ++r) {
    if (t->kv_len[r] == 0) return fail("sparse row %u: kv_len is 0; every row needs at least one KV row", r);
    if (t->width[r] == 0) return fail("sparse row %u: width is 0; every row attends to at least one slot", r);
    p->q_rows = std::max<uint64_t>(p->q_rows, uint64_t(t->q_row[r]) + 1);
    p->index_end = std::max<uint64_t>(p->index_end, uint64_t(t->index_offset[r]) + t->width[r]);
    p->slot_base[r] = p->slots;
    p->slots += t->width[r];
    p->chunks[r] = div_up(t->width[r], ds::kAttnChunk);
    p->max_chunks = std::max(p->max_chunks, p->chunks[r]);
  }
  // Every row gets room for the call's largest chunk count, so that a row's
  // statistics and partials start at r * max_chunks chunks: the combine finds
  // them from its row index alone.
  for (uint32_t r = 0; r < t->rows; ++r) {
    p->stat_base[r] = uint64_t(r) * p->max_chunks * ds::kHeads;
    p->part_base[r] = uint64_t(r) * p->max_chunks * ds::kHeads * ds::kDim;
  }
  p->stat_elems = uint64_t(t->rows) * p->max_chunks * ds::kHeads;
  p->part_elems = uint64_t(t->rows) * p->max_chunks * ds::kHeads * ds::kDim;
  // Each row writes its own query row of the output: no two may share one.
  uint64_t qr[DS_ROWS_MAX];
  for (uint32_t r = 0; r < t->rows; ++r) qr[r] = t->q_row[r];
  uint32_t a, b;
  if (overlapping_pair(qr, 1, t->rows, &a, &b))
    return fail("sparse rows %u and %u both use q_row %u (each row writes its own output row)", a, b, t->q_row[a]);
  return DS_OK;
}

// Attention workspace: f32x4 chunk statistics, then the f32 chunk outputs,
// each with max_chunks chunks per row.
uint64_t attn_stat_bytes(const SparsePlan &p) { return align256(p.stat_elems * 16); }
uint64_t attn_workspace_bytes(const SparsePlan &p) {
  return attn_stat_bytes(p) + align256(p.part_elems * sizeof(float));
}

ds_status need(const void *ptr, const char *name) {
  return ptr ? DS_OK : fail("%s must not be null", name);
}
ds_status cap(uint64_t have, uint64_t want, const char *name, const char *unit) {
  if (have < want) return fail("%s holds %llu %s, needs %llu", name, (unsigned long long)have, unit,
                               (unsigned long long)want);
  return DS_OK;
}

#define DS_TRY(x)                   \
  do {                              \
    const ds_status st_ = (x);      \
    if (st_ != DS_OK) return st_;   \
  } while (0)

// Operand checks shared by the indexer entry points.
ds_status check_indexer_operands(const ds_indexer_rows *rows, const IndexerPlan &p, const void *q, size_t q_elems,
                                 const float *weights, size_t weights_elems, const float *scores,
                                 size_t scores_elems) {
  DS_TRY(need(q, "indexer q"));
  DS_TRY(need(weights, "indexer weights"));
  DS_TRY(need(scores, "indexer scores"));
  for (uint32_t r = 0; r < p.rows; ++r) {
    if (!rows->keys[r]) return fail("indexer row %u: keys must not be null", r);
    DS_TRY(cap(rows->keys_elems[r], uint64_t(rows->kv_len[r]) * DS_INDEXER_DIM, "indexer kv", "elements"));
  }
  DS_TRY(cap(q_elems, p.q_rows * DS_HEADS * DS_INDEXER_DIM, "indexer q", "elements"));
  DS_TRY(cap(weights_elems, p.q_rows * DS_HEADS, "indexer weights", "elements"));
  DS_TRY(cap(scores_elems, p.rows * p.max_kv, "indexer scores", "elements"));
  return DS_OK;
}

// The calling thread's armed indexer timing buffer (ds_rows_time_next_indexer),
// taken by its next indexer launch.
thread_local uint64_t *t_timer_stamps = nullptr;
thread_local size_t t_timer_elems = 0;

// Indexer launch; with cand/floors set, also the fused top-k stage.
ds_status launch_indexer(const ds_indexer_rows *rows, const IndexerPlan &p, const void *q, const float *weights,
                         float *scores, uint64_t *cand, uint64_t *floors, void *stream) {
  ds::IndexerArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.w = weights;
  a.scores = scores;
  a.score_stride = p.max_kv;
  a.rows = p.rows;
  a.cand = cand;
  a.floors = floors;
  // Slot y of the grid takes row order[y]. The fused stage keeps the rows in
  // order (its candidate and floor layout is per 1024-key block, row after
  // row). The plain kernel takes the rows longest first: workgroups are
  // dispatched in grid order, and with a long row last its workgroups waited
  // behind every short row's (mostly empty) grid row; at workload 3 (rows of
  // 1 .. 131072 keys) the long row's last workgroup started 9.4 us into the
  // kernel.
  uint32_t order[ds::kRowsMax];
  for (uint32_t r = 0; r < p.rows; ++r) order[r] = r;
  if (cand != nullptr) {
    a.keys_per_block = kIndexerKeysPerBlock;
    for (uint32_t r = 0; r <= ds::kRowsMax; ++r) a.blk_begin[r] = p.blk_begin[r];
  } else {
    a.keys_per_block = plain_keys_per_block(rows, p.rows);
    std::stable_sort(order, order + p.rows,
                     [&](uint32_t x, uint32_t y) { return rows->kv_len[x] > rows->kv_len[y]; });
    for (uint32_t y = 0; y < ds::kRowsMax; ++y)
      a.blk_begin[y + 1] = a.blk_begin[y] + (y < p.rows ? div_up(rows->kv_len[order[y]], a.keys_per_block) : 0);
  }
  for (uint32_t y = 0; y < p.rows; ++y) {
    const uint32_t r = order[y];
    a.keys[y] = static_cast<const uint16_t *>(rows->keys[r]);
    a.kv_len[y] = rows->kv_len[r];
    a.visible[y] = p.visible[r];
    a.q_row[y] = rows->q_row[r];
    a.score_row[y] = r;
  }
  uint32_t max_row_blocks = 1;
  for (uint32_t r = 0; r < p.rows; ++r) max_row_blocks = std::max(max_row_blocks, a.blk_begin[r + 1] - a.blk_begin[r]);
  // The plain kernel takes a compact grid (one workgroup per block) when the
  // (blocks of the longest row) x rows grid would be more than twice its
  // blocks, i.e. mostly empty workgroups.
  const uint64_t blocks = a.blk_begin[ds::kRowsMax];
  const bool compact = cand == nullptr && uint64_t(max_row_blocks) * p.rows > 2 * blocks;
  if (t_timer_stamps != nullptr) {
    const uint64_t wgs = compact ? blocks : uint64_t(max_row_blocks) * p.rows;
    const uint64_t need_elems = wgs * ds::kTimerStamps;
    if (t_timer_elems < need_elems)
      return fail("the indexer timing buffer holds %zu entries; this launch's %llu workgroups need %llu",
                  t_timer_elems, static_cast<unsigned long long>(wgs), static_cast<unsigned long long>(need_elems));
    a.stamps = t_timer_stamps;
    t_timer_stamps = nullptr;
    t_timer_elems = 0;
  }
  const hipError_t e = ds::launch_indexer_score(a, max_row_blocks, cand != nullptr ? fused_wave_cand(p) : 0, compact,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DS_OK : hip_fail(e, "indexer score launch");
}

// First-level input of the top-k levels: the scores (lists == nullptr;
// count = visible keys) or the fused indexer's candidate lists (count and
// base per row, with the block floors to check on the final level).
struct TopkInput {
  const uint64_t *lists = nullptr;
  const uint64_t *floors = nullptr;
  uint32_t count[ds::kRowsMax] = {};
  uint64_t base[ds::kRowsMax] = {};
  uint32_t room = 0;          // lists: entries of room per row (row r's at r * room)
  uint32_t floor_room = 0;    // floors of room per row
};

// The fused indexer's candidates: 4 waves x C slots per 1024-key block, row r
// from block r * room (room = the widest row's blocks).
TopkInput fused_input(const IndexerPlan &p, const uint64_t *cand, const uint64_t *floors) {
  TopkInput in{};
  in.lists = cand;
  in.floors = floors;
  const uint32_t per_block = ds::kIdxFloors * fused_wave_cand(p);
  const uint32_t room = fused_room_blocks(p);
  in.room = room * per_block;
  in.floor_room = room * ds::kIdxFloors;
  for (uint32_t r = 0; r < p.rows; ++r) {
    in.count[r] = (p.blk_begin[r + 1] - p.blk_begin[r]) * per_block;
    in.base[r] = uint64_t(r) * in.room;
  }
  return in;
}

// Selection levels until every row has one list; the last writes indices.
// With attn set, the pass over lists in which every row that is still
// selecting reaches its final level runs inside the attention's workgroups
// instead (rows that finished in earlier passes read their indices there),
// followed by the attention's combine, and *attn_done says so.
ds_status run_topk_levels(const ds_indexer_rows *rows, const IndexerPlan &p, const float *scores,
                          const TopkInput &in, uint64_t *bank0, uint64_t *bank1, int32_t *indices, void *stream,
                          const ds::AttnArgs *attn = nullptr, uint32_t attn_chunks = 0, bool *attn_done = nullptr) {
  uint64_t *bank[2] = {bank0, bank1};
  const bool from_lists = in.lists != nullptr;
  uint32_t count[ds::kRowsMax] = {}, chunks[ds::kRowsMax] = {};
  uint64_t in_base[ds::kRowsMax] = {};
  bool done[ds::kRowsMax] = {};
  for (uint32_t r = 0; r < p.rows; ++r) {
    count[r] = in.count[r];
    in_base[r] = in.base[r];
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (uint32_t level = 0;; ++level) {
    ds::TopkLevelArgs a{};
    a.scores = scores;
    a.score_stride = p.max_kv;
    a.in = level == 0 ? in.lists : bank[(level - 1) & 1];
    a.out = bank[level & 1];
    a.indices = indices;
    a.rows = p.rows;
    a.from_scores = (level == 0 && !from_lists) ? 1 : 0;
    a.floors = in.floors;
    a.list_room = level == 0 ? in.room : 0;   // later levels' lists sit one row after another
    a.floor_room = in.floor_room;
    // Candidates per thread, and so the chunk size: the smallest of 4, 8 and
    // 16 that holds every row still selecting, which makes this the final
    // level; otherwise chunks of scores (see scores_per_thread) or of 8192
    // list keys.
    uint32_t max_count = 0;
    for (uint32_t r = 0; r < p.rows; ++r)
      if (!done[r]) max_count = std::max(max_count, count[r]);
    if (a.from_scores) {
      a.per_thread = scores_per_thread(max_count);   // (the banks are sized by the same rule)
    } else {
      a.per_thread = ds::kTopkPerThreadLater;
      for (uint32_t per : {4u, 8u, 16u})
        if (max_count <= ds::kTopkThreads * per) { a.per_thread = per; break; }
    }
    for (uint32_t r = 0; r < p.rows; ++r)
      if (!done[r]) chunks[r] = std::max<uint32_t>(1, div_up(count[r], uint64_t(ds::kTopkThreads) * a.per_thread));
    uint32_t blocks = 0;
    uint64_t out_elems = 0;
    for (uint32_t r = 0; r < ds::kRowsMax; ++r) {
      a.blk_begin[r] = blocks;
      if (r >= p.rows) continue;
      a.offset[r] = rows->offset[r];
      a.out_offset[r] = rows->output_offset[r];   // (also where a finished row's indices are)
      if (done[r]) continue;
      a.count[r] = count[r];
      a.in_base[r] = in_base[r];
      a.out_base[r] = out_elems;
      if (chunks[r] == 1) {
        a.final_mask |= 1u << r;
        if (from_lists) {
          a.check_mask |= 1u << r;
          a.floor_begin[r] = uint64_t(r) * in.floor_room;
          a.floor_count[r] = (p.blk_begin[r + 1] - p.blk_begin[r]) * ds::kIdxFloors;
          a.fallback_count[r] = p.visible[r];
        }
      } else {
        out_elems += uint64_t(chunks[r]) * DS_TOP_K;
      }
      blocks += chunks[r];
    }
    a.blk_begin[ds::kRowsMax] = blocks;
    bool every_row_final = true;
    for (uint32_t r = 0; r < p.rows; ++r) every_row_final &= done[r] || chunks[r] == 1;
    if (attn && !a.from_scores && every_row_final) {
      hipError_t e = ds::launch_topk_attn(a, *attn, attn_chunks, s);
      if (e != hipSuccess) return hip_fail(e, "top-k and attention launch");
      e = ds::launch_attn_combine(*attn, s);
      if (e != hipSuccess) return hip_fail(e, "attention combine launch");
      *attn_done = true;
      return DS_OK;
    }
    const hipError_t e = ds::launch_topk_level(a, blocks, s);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    bool all = true;
    for (uint32_t r = 0; r < p.rows; ++r) {
      if (done[r]) continue;
      if (chunks[r] == 1) { done[r] = true; continue; }
      all = false;
      in_base[r] = a.out_base[r];
      count[r] = chunks[r] * DS_TOP_K;
    }
    if (all) break;
  }
  return DS_OK;
}

}  // namespace

ds_status ds::record_error(ds_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = std::string("ds_rows: ") + buf;
  return st;
}

extern "C" {


size_t ds_rows_scores_elems(const ds_indexer_rows *rows) {
  IndexerPlan p;
  if (check_indexer(rows, &p) != DS_OK) return 0;
  return p.rows * p.max_kv;
}

size_t ds_rows_topk_workspace_bytes(const ds_indexer_rows *rows) {
  IndexerPlan p;
  if (check_indexer(rows, &p) != DS_OK) return 0;
  return topk_workspace_bytes(p);
}

size_t ds_rows_gathered_elems(const ds_sparse_rows *rows) {
  SparsePlan p;
  if (check_sparse(rows, &p) != DS_OK) return 0;
  return p.slots * DS_HEAD_DIM;
}

size_t ds_rows_mask_elems(const ds_sparse_rows *rows) {
  SparsePlan p;
  if (check_sparse(rows, &p) != DS_OK) return 0;
  return p.slots;
}

size_t ds_rows_attn_workspace_bytes(const ds_sparse_rows *rows) {
  SparsePlan p;
  if (check_sparse(rows, &p) != DS_OK) return 0;
  return attn_workspace_bytes(p);
}

ds_status ds_rows_indexer_score(const ds_indexer_rows *rows, const void *q, size_t q_elems, const float *weights,
                                size_t weights_elems, float *scores, size_t scores_elems, void *stream) {
  IndexerPlan p;
  DS_TRY(check_indexer(rows, &p));
  DS_TRY(check_indexer_operands(rows, p, q, q_elems, weights, weights_elems, scores, scores_elems));
  DS_TRY(check_device());
  return launch_indexer(rows, p, q, weights, scores, nullptr, nullptr, stream);
}

ds_status ds_rows_topk(const ds_indexer_rows *rows, const float *scores, size_t scores_elems, void *workspace,
                       size_t workspace_bytes, int32_t *indices, size_t indices_elems, void *stream) {
  IndexerPlan p;
  DS_TRY(check_indexer(rows, &p));
  DS_TRY(need(scores, "indexer scores"));
  DS_TRY(need(indices, "indexer output"));
  const uint64_t ws = topk_workspace_bytes(p);
  if (ws) DS_TRY(need(workspace, "indexer top-k scratch"));
  DS_TRY(cap(scores_elems, p.rows * p.max_kv, "indexer scores", "elements"));
  DS_TRY(cap(workspace_bytes, ws, "indexer top-k scratch", "bytes"));
  DS_TRY(cap(indices_elems, p.indices_end, "indexer output", "elements"));
  DS_TRY(check_device());

  TopkInput in{};
  for (uint32_t r = 0; r < p.rows; ++r) in.count[r] = p.visible[r];
  uint64_t *bank = static_cast<uint64_t *>(workspace);
  return run_topk_levels(rows, p, scores, in, bank, bank + p.topk_bank, indices, stream);
}

size_t ds_rows_indexer_topk_workspace_bytes(const ds_indexer_rows *rows) {
  IndexerPlan p;
  if (check_indexer(rows, &p) != DS_OK) return 0;
  return indexer_topk_workspace_bytes(p);
}

ds_status ds_rows_indexer_candidates(const ds_indexer_rows *rows, const void *q, size_t q_elems, const float *weights,
                                     size_t weights_elems, float *scores, size_t scores_elems, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  IndexerPlan p;
  DS_TRY(check_indexer(rows, &p));
  DS_TRY(check_indexer_operands(rows, p, q, q_elems, weights, weights_elems, scores, scores_elems));
  DS_TRY(need(workspace, "indexer top-k workspace"));
  DS_TRY(cap(workspace_bytes, indexer_topk_workspace_bytes(p), "indexer top-k workspace", "bytes"));
  DS_TRY(check_device());
  char *ws = static_cast<char *>(workspace);
  return launch_indexer(rows, p, q, weights, scores, reinterpret_cast<uint64_t *>(ws),
                        reinterpret_cast<uint64_t *>(ws + fused_cand_bytes(p)), stream);
}

ds_status ds_rows_indexer_topk(const ds_indexer_rows *rows, const void *q, size_t q_elems, const float *weights,
                               size_t weights_elems, float *scores, size_t scores_elems, void *workspace,
                               size_t workspace_bytes, int32_t *indices, size_t indices_elems, void *stream) {
  IndexerPlan p;
  DS_TRY(check_indexer(rows, &p));
  DS_TRY(check_indexer_operands(rows, p, q, q_elems, weights, weights_elems, scores, scores_elems));
  DS_TRY(need(workspace, "indexer top-k workspace"));
  DS_TRY(need(indices, "indexer output"));
  DS_TRY(cap(workspace_bytes, indexer_topk_workspace_bytes(p), "indexer top-k workspace", "bytes"));
  DS_TRY(cap(indices_elems, p.indices_end, "indexer output", "elements"));
  DS_TRY(check_device());

  if (!fused_rows(p)) {
    DS_TRY(launch_indexer(rows, p, q, weights, scores, nullptr, nullptr, stream));
    TopkInput in{};
    for (uint32_t r = 0; r < p.rows; ++r) in.count[r] = p.visible[r];
    uint64_t *bank = static_cast<uint64_t *>(workspace);
    return run_topk_levels(rows, p, scores, in, bank, bank + p.topk_bank, indices, stream);
  }
  char *ws = static_cast<char *>(workspace);
  uint64_t *cand = reinterpret_cast<uint64_t *>(ws);
  uint64_t *floors = reinterpret_cast<uint64_t *>(ws + fused_cand_bytes(p));
  uint64_t *bank = reinterpret_cast<uint64_t *>(ws + fused_cand_bytes(p) + fused_floor_bytes(p));
  DS_TRY(launch_indexer(rows, p, q, weights, scores, cand, floors, stream));
  return run_topk_levels(rows, p, scores, fused_input(p, cand, floors), bank, bank + p.fused_bank, indices, stream);
}

ds_status ds_rows_gather(const ds_sparse_rows *rows, const int32_t *indices, size_t indices_elems, void *gathered,
                         size_t gathered_elems, void *mask, size_t mask_elems, uint32_t *invalid,
                         size_t invalid_elems, void *stream) {
  SparsePlan p;
  DS_TRY(check_sparse(rows, &p));
  DS_TRY(need(indices, "indices"));
  DS_TRY(need(gathered, "gathered_kv"));
  DS_TRY(need(mask, "mask"));
  DS_TRY(need(invalid, "invalid"));
  for (uint32_t r = 0; r < p.rows; ++r) {
    if (!rows->kv[r]) return fail("sparse row %u: kv must not be null", r);
    DS_TRY(cap(rows->kv_elems[r], uint64_t(rows->kv_len[r]) * DS_HEAD_DIM, "kv", "elements"));
  }
  DS_TRY(cap(indices_elems, p.index_end, "indices", "elements"));
  DS_TRY(cap(gathered_elems, p.slots * DS_HEAD_DIM, "gathered_kv", "elements"));
  DS_TRY(cap(mask_elems, p.slots, "mask", "elements"));
  DS_TRY(cap(invalid_elems, p.rows, "invalid", "elements"));
  DS_TRY(check_device());

  ds::GatherArgs a{};
  a.indices = indices;
  a.gathered = static_cast<uint16_t *>(gathered);
  a.mask = static_cast<uint16_t *>(mask);
  a.invalid = invalid;
  a.rows = p.rows;
  uint32_t max_row_blocks = 1;
  for (uint32_t r = 0; r < p.rows; ++r) {
    a.kv[r] = static_cast<const uint16_t *>(rows->kv[r]);
    a.kv_len[r] = rows->kv_len[r];
    a.width[r] = rows->width[r];
    a.index_offset[r] = rows->index_offset[r];
    a.slot_base[r] = p.slot_base[r];
    max_row_blocks = std::max(max_row_blocks, div_up(rows->width[r], ds::kGatherSlotsPerBlock));
  }
  const hipError_t e = ds::launch_gather(a, max_row_blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DS_OK : hip_fail(e, "gather launch");
}

}  // extern "C"

namespace {

// Both attention entry points after their own operand checks.
ds::AttnArgs attention_args(const ds_sparse_rows *rows, const SparsePlan &p, const void *q, const float *sinks,
                            const void *gathered, const void *mask, const uint32_t *invalid,
                            const int32_t *indices, float scale, void *workspace, float *out) {
  ds::AttnArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.sinks = sinks;
  a.gathered = static_cast<const uint16_t *>(gathered);
  a.mask = static_cast<const uint16_t *>(mask);
  a.invalid = invalid;
  a.indices = indices;
  char *ws = static_cast<char *>(workspace);
  a.stats = reinterpret_cast<float4 *>(ws);
  a.opart = reinterpret_cast<float *>(ws + attn_stat_bytes(p));
  a.out = out;
  a.scale = scale;
  a.rows = p.rows;
  a.row_chunks = p.max_chunks;
  for (uint32_t r = 0; r < p.rows; ++r) {
    a.kv[r] = static_cast<const uint16_t *>(rows->kv[r]);
    a.kv_len[r] = rows->kv_len[r];
    a.index_offset[r] = rows->index_offset[r];
    a.width[r] = rows->width[r];
    a.chunks[r] = p.chunks[r];
    a.q_row[r] = rows->q_row[r];
    a.slot_base[r] = p.slot_base[r];
    a.stat_base[r] = p.stat_base[r];
    a.part_base[r] = p.part_base[r];
  }
  return a;
}

ds_status launch_attention(const ds_sparse_rows *rows, const SparsePlan &p, bool direct, const void *q,
                           const float *sinks, const void *gathered, const void *mask, const uint32_t *invalid,
                           const int32_t *indices, float scale, void *workspace, float *out, void *stream) {
  const ds::AttnArgs a = attention_args(rows, p, q, sinks, gathered, mask, invalid, indices, scale, workspace, out);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = ds::launch_attn_chunks(a, direct, p.max_chunks, s);
  if (e != hipSuccess) return hip_fail(e, "attention chunk launch");
  e = ds::launch_attn_combine(a, s);
  return e == hipSuccess ? DS_OK : hip_fail(e, "attention combine launch");
}

ds_status check_attention_common(const SparsePlan &p, const void *q, size_t q_elems, const float *sinks,
                                 size_t sinks_elems, float scale, void *workspace, size_t workspace_bytes,
                                 float *out, size_t out_elems) {
  if (!(std::isfinite(scale) && scale > 0.0f)) return fail("scale %g is not a finite value above 0", double(scale));
  DS_TRY(need(q, "q"));
  DS_TRY(need(sinks, "sinks"));
  DS_TRY(need(workspace, "attention workspace"));
  DS_TRY(need(out, "output"));
  DS_TRY(cap(q_elems, p.q_rows * DS_HEADS * DS_HEAD_DIM, "q", "elements"));
  DS_TRY(cap(out_elems, p.q_rows * DS_HEADS * DS_HEAD_DIM, "output", "elements"));
  DS_TRY(cap(sinks_elems, DS_HEADS, "sinks", "elements"));
  DS_TRY(cap(workspace_bytes, attn_workspace_bytes(p), "attention workspace", "bytes"));
  return DS_OK;
}

}  // namespace

extern "C" {

ds_status ds_rows_sparse_attn(const ds_sparse_rows *rows, const void *q, size_t q_elems, const float *sinks,
                              size_t sinks_elems, const void *gathered, size_t gathered_elems, const void *mask,
                              size_t mask_elems, const uint32_t *invalid, size_t invalid_elems, float scale,
                              void *workspace, size_t workspace_bytes, float *out, size_t out_elems, void *stream) {
  SparsePlan p;
  DS_TRY(check_sparse(rows, &p));
  DS_TRY(check_attention_common(p, q, q_elems, sinks, sinks_elems, scale, workspace, workspace_bytes, out,
                                out_elems));
  DS_TRY(need(gathered, "gathered_kv"));
  DS_TRY(need(mask, "mask"));
  DS_TRY(cap(gathered_elems, p.slots * DS_HEAD_DIM, "gathered_kv", "elements"));
  DS_TRY(cap(mask_elems, p.slots, "mask", "elements"));
  DS_TRY(need(invalid, "invalid"));
  DS_TRY(cap(invalid_elems, p.rows, "invalid", "elements"));
  DS_TRY(check_device());
  return launch_attention(rows, p, false, q, sinks, gathered, mask, invalid, nullptr, scale, workspace, out, stream);
}

ds_status ds_rows_sparse_attn_direct(const ds_sparse_rows *rows, const void *q, size_t q_elems, const float *sinks,
                                     size_t sinks_elems, const int32_t *indices, size_t indices_elems, float scale,
                                     void *workspace, size_t workspace_bytes, float *out, size_t out_elems,
                                     void *stream) {
  SparsePlan p;
  DS_TRY(check_sparse(rows, &p));
  DS_TRY(check_attention_common(p, q, q_elems, sinks, sinks_elems, scale, workspace, workspace_bytes, out,
                                out_elems));
  DS_TRY(need(indices, "indices"));
  for (uint32_t r = 0; r < p.rows; ++r) {
    if (!rows->kv[r]) return fail("sparse row %u: kv must not be null", r);
    DS_TRY(cap(rows->kv_elems[r], uint64_t(rows->kv_len[r]) * DS_HEAD_DIM, "kv", "elements"));
  }
  DS_TRY(cap(indices_elems, p.index_end, "indices", "elements"));
  DS_TRY(check_device());
  return launch_attention(rows, p, true, q, sinks, nullptr, nullptr, nullptr, indices, scale, workspace, out, stream);
}

ds_status ds_rows_indexer_topk_attn(const ds_indexer_rows *irows, const ds_sparse_rows *srows, const void *idx_q,
                                    size_t idx_q_elems, const float *weights, size_t weights_elems, float *scores,
                                    size_t scores_elems, void *idx_workspace, size_t idx_workspace_bytes,
                                    int32_t *indices, size_t indices_elems, const void *q, size_t q_elems,
                                    const float *sinks, size_t sinks_elems, float scale, void *attn_workspace,
                                    size_t attn_workspace_bytes, float *out, size_t out_elems, void *stream) {
  IndexerPlan p;
  DS_TRY(check_indexer(irows, &p));
  DS_TRY(check_indexer_operands(irows, p, idx_q, idx_q_elems, weights, weights_elems, scores, scores_elems));
  DS_TRY(need(idx_workspace, "indexer top-k workspace"));
  DS_TRY(need(indices, "indexer output"));
  DS_TRY(cap(idx_workspace_bytes, indexer_topk_workspace_bytes(p), "indexer top-k workspace", "bytes"));
  DS_TRY(cap(indices_elems, p.indices_end, "indexer output", "elements"));
  SparsePlan sp;
  DS_TRY(check_sparse(srows, &sp));
  DS_TRY(check_attention_common(sp, q, q_elems, sinks, sinks_elems, scale, attn_workspace, attn_workspace_bytes, out,
                                out_elems));
  for (uint32_t r = 0; r < sp.rows; ++r) {
    if (!srows->kv[r]) return fail("sparse row %u: kv must not be null", r);
    DS_TRY(cap(srows->kv_elems[r], uint64_t(srows->kv_len[r]) * DS_HEAD_DIM, "kv", "elements"));
  }
  if (sp.rows != p.rows) return fail("the indexer table has %u rows but the sparse table %u", p.rows, sp.rows);
  for (uint32_t r = 0; r < p.rows; ++r) {
    if (srows->width[r] > DS_TOP_K)
      return fail("sparse row %u: width %u is above the %d selected slots", r, srows->width[r], DS_TOP_K);
    if (srows->index_offset[r] != irows->output_offset[r])
      return fail("sparse row %u: index_offset %u differs from the indexer row's output_offset %u", r,
                  srows->index_offset[r], irows->output_offset[r]);
  }
  DS_TRY(check_device());

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const ds::AttnArgs a =
      attention_args(srows, sp, q, sinks, nullptr, nullptr, nullptr, indices, scale, attn_workspace, out);
  ds::TopkLevelArgs t{};
  t.scores = scores;
  t.score_stride = p.max_kv;
  t.indices = indices;
  t.rows = p.rows;
  for (uint32_t r = 0; r < p.rows; ++r) {
    t.offset[r] = irows->offset[r];
    t.out_offset[r] = irows->output_offset[r];
    t.final_mask |= 1u << r;
    t.blk_begin[r] = r;
  }
  for (uint32_t r = p.rows; r <= ds::kRowsMax; ++r) t.blk_begin[r] = p.rows;

  // Rows too short for the indexer's first stage whose visible scores all fit
  // one selection chunk (at most 16384): the score kernel, then the one level
  // from the scores inside the attention's workgroups, with the chunk size
  // ds_rows_indexer_topk would take.
  uint32_t max_visible = 0;
  for (uint32_t r = 0; r < p.rows; ++r) max_visible = std::max(max_visible, p.visible[r]);
  if (!fused_rows(p) && max_visible <= ds::kTopkThreads * 16) {
    DS_TRY(launch_indexer(irows, p, idx_q, weights, scores, nullptr, nullptr, stream));
    t.from_scores = 1;
    t.per_thread = 16;
    for (uint32_t per : {4u, 8u})
      if (max_visible <= ds::kTopkThreads * per) { t.per_thread = per; break; }
    for (uint32_t r = 0; r < p.rows; ++r) t.count[r] = p.visible[r];
    hipError_t e = ds::launch_topk_attn(t, a, sp.max_chunks, s);
    if (e != hipSuccess) return hip_fail(e, "top-k and attention launch");
    e = ds::launch_attn_combine(a, s);
    return e == hipSuccess ? DS_OK : hip_fail(e, "attention combine launch");
  }

  // Otherwise ds_rows_indexer_topk's kernels (the fused indexer and selection
  // passes over its candidates when every row is long enough, else the score
  // kernel and passes over the scores), with the last selection pass inside
  // the attention's workgroups whenever it is a pass over lists; when the
  // only pass is over the scores, ds_rows_sparse_attn_direct follows.
  TopkInput in{};
  uint64_t *bank0, *bank1;
  if (fused_rows(p)) {
    char *ws = static_cast<char *>(idx_workspace);
    uint64_t *cand = reinterpret_cast<uint64_t *>(ws);
    uint64_t *floors = reinterpret_cast<uint64_t *>(ws + fused_cand_bytes(p));
    bank0 = reinterpret_cast<uint64_t *>(ws + fused_cand_bytes(p) + fused_floor_bytes(p));
    bank1 = bank0 + p.fused_bank;
    DS_TRY(launch_indexer(irows, p, idx_q, weights, scores, cand, floors, stream));
    in = fused_input(p, cand, floors);
  } else {
    bank0 = static_cast<uint64_t *>(idx_workspace);
    bank1 = bank0 + p.topk_bank;
    DS_TRY(launch_indexer(irows, p, idx_q, weights, scores, nullptr, nullptr, stream));
    for (uint32_t r = 0; r < p.rows; ++r) in.count[r] = p.visible[r];
  }
  bool attn_done = false;
  DS_TRY(run_topk_levels(irows, p, scores, in, bank0, bank1, indices, stream, &a, sp.max_chunks, &attn_done));
  if (attn_done) return DS_OK;
  return ds_rows_sparse_attn_direct(srows, q, q_elems, sinks, sinks_elems, indices, indices_elems, scale,
                                    attn_workspace, attn_workspace_bytes, out, out_elems, stream);
}

ds_status ds_rows_time_next_indexer(uint64_t *stamps, size_t stamps_elems) {
  DS_TRY(need(stamps, "indexer timing stamps"));
  t_timer_stamps = stamps;
  t_timer_elems = stamps_elems;
  return DS_OK;
}

ds_status ds_rows_wall_clock_khz(int *khz) {
  DS_TRY(need(khz, "khz"));
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ds::record_error(DS_ERR_DEVICE, "no current HIP device");
  const hipError_t e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return e == hipSuccess ? DS_OK : ds::record_error(DS_ERR_DEVICE, "the wall clock rate is unavailable (%s)",
                                                     hipGetErrorString(e));
}

const char *ds_rows_last_error(void) { return g_error.c_str(); }

const char *ds_rows_version(void) { return "ds_rows 0.1.0 (gfx950)"; }

}  // extern "C"

// ---------------------------------------------------------------- compressor
namespace {

bool compressor_shape_ok(uint32_t ratio, uint32_t head_dim) {
  return (ratio == 4 && (head_dim == 128 || head_dim == 512)) || (ratio == 128 && head_dim == 512);
}

ds_status compressor_shape_error(uint32_t ratio, uint32_t head_dim) {
  return fail("compressor shape (ratio %u, head_dim %u) is unsupported; supported are ratio 4 with head_dim 128 "
              "or 512, and ratio 128 with head_dim 512", ratio, head_dim);
}

}  // namespace

extern "C" {

size_t ds_rows_compressor_state_elems(uint32_t ratio, uint32_t head_dim) {
  if (!compressor_shape_ok(ratio, head_dim)) {
    compressor_shape_error(ratio, head_dim);
    return 0;
  }
  const uint64_t coff = ratio == 4 ? 2 : 1;
  return static_cast<size_t>(coff * ratio * coff * head_dim);
}

ds_status ds_rows_compressor(const ds_compressor_rows *rows, uint32_t ratio, uint32_t head_dim, float epsilon,
                             const float *kv, size_t kv_elems, const float *score, size_t score_elems,
                             const float *ape, size_t ape_elems, const float *norm, size_t norm_elems, void *output,
                             size_t output_elems, void *stream) {
  if (!rows) return fail("compressor row table is null");
  DS_TRY(check_row_count(rows->rows));
  if (!compressor_shape_ok(ratio, head_dim)) return compressor_shape_error(ratio, head_dim);
  if (!(std::isfinite(epsilon) && epsilon > 0.0f))
    return fail("compressor epsilon %g is not a finite value above 0", double(epsilon));
  const uint64_t coff = ratio == 4 ? 2 : 1;
  const uint64_t proj = coff * head_dim;
  const uint64_t state = coff * ratio * proj;
  const uint32_t n = rows->rows;
  for (uint32_t r = 0; r < n; ++r) {
    // start_pos 0 would have no earlier token; the largest position leaves no
    // next one.
    if (rows->start_pos[r] < 1 || rows->start_pos[r] > UINT32_MAX - 1)
      return fail("compressor row %u: start_pos %u is outside [1, 2^32 - 2]", r, rows->start_pos[r]);
    if (!rows->kv_state[r]) return fail("compressor row %u: kv_state must not be null", r);
    if (!rows->score_state[r]) return fail("compressor row %u: score_state must not be null", r);
    DS_TRY(cap(rows->kv_state_elems[r], state, "kv_state", "elements"));
    DS_TRY(cap(rows->score_state_elems[r], state, "score_state", "elements"));
  }
  // Every state buffer of every row is written: all 2n byte ranges must be
  // disjoint (kv states are buffers 0..n-1, score states n..2n-1).
  {
    std::pair<uintptr_t, uint32_t> b[2 * DS_ROWS_MAX];
    for (uint32_t r = 0; r < n; ++r) {
      b[r] = {reinterpret_cast<uintptr_t>(rows->kv_state[r]), r};
      b[n + r] = {reinterpret_cast<uintptr_t>(rows->score_state[r]), n + r};
    }
    std::sort(b, b + 2 * n);
    for (uint32_t i = 1; i < 2 * n; ++i)
      if (b[i].first < b[i - 1].first + state * sizeof(float))
        return fail("compressor state buffers %u and %u share memory (buffers 0..rows-1 are the kv states, "
                    "rows..2 rows-1 the score states)", std::min(b[i - 1].second, b[i].second),
                    std::max(b[i - 1].second, b[i].second));
  }
  DS_TRY(need(kv, "kv"));
  DS_TRY(need(score, "score"));
  DS_TRY(need(ape, "ape"));
  DS_TRY(need(norm, "norm"));
  DS_TRY(need(output, "output"));
  DS_TRY(cap(kv_elems, n * proj, "kv", "elements"));
  DS_TRY(cap(score_elems, n * proj, "score", "elements"));
  DS_TRY(cap(ape_elems, ratio * proj, "ape", "elements"));
  DS_TRY(cap(norm_elems, head_dim, "norm", "elements"));
  DS_TRY(cap(output_elems, uint64_t(n) * head_dim, "output", "elements"));
  DS_TRY(check_device());

  ds::CompressorArgs a{};
  a.kv = kv;
  a.score = score;
  a.ape = ape;
  a.norm = norm;
  a.out = static_cast<uint16_t *>(output);
  for (uint32_t r = 0; r < n; ++r) {
    a.kv_state[r] = rows->kv_state[r];
    a.score_state[r] = rows->score_state[r];
    a.start_pos[r] = rows->start_pos[r];
  }
  a.rows = n;
  a.ratio = ratio;
  a.head_dim = head_dim;
  a.eps = epsilon;
  const hipError_t e = ds::launch_compressor(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DS_OK : hip_fail(e, "compressor launch");
}

}  // extern "C"

// ------------------------------------------------------- multi-query indexer
namespace {

constexpr uint32_t kMqKeysPerBlock = 1024;

struct MqPlan {
  uint32_t rows = 0;
  uint64_t max_kv = 0;
  uint64_t q_rows = 0;                      // max q_row + query_len
  uint32_t blk_begin[ds::kRowsMax + 1] = {};
};

// The row-table checks that concern scoring (rows, kv_len, positions and the
// causal length of the last query); offsets and output offsets are not used.
ds_status check_mq(const ds_indexer_rows *t, uint32_t query_len, MqPlan *p) {
  if (!t) return fail("indexer row table is null");
  DS_TRY(check_row_count(t->rows));
  if (query_len < 1 || query_len > uint32_t(ds::kMqMaxQueries))
    return fail("query_len %u is outside [1, %d]", query_len, ds::kMqMaxQueries);
  p->rows = t->rows;
  for (uint32_t r = 0; r < t->rows; ++r) {
    if (uint64_t(t->start_pos[r]) + query_len > UINT32_MAX)
      return fail("indexer row %u: the last query's position start_pos %u + %u is past 2^32 - 2", r,
                  t->start_pos[r], query_len - 1);
    // The row's fields as for one query at the last query's position; the
    // offset is not used by the scores.
    uint32_t visible;
    DS_TRY(check_indexer_row(r, t->kv_len[r], t->start_pos[r] + query_len - 1, 0, &visible));
    p->max_kv = std::max<uint64_t>(p->max_kv, t->kv_len[r]);
    p->q_rows = std::max<uint64_t>(p->q_rows, uint64_t(t->q_row[r]) + query_len);
    p->blk_begin[r + 1] = p->blk_begin[r] + div_up(t->kv_len[r], kMqKeysPerBlock);
  }
  for (uint32_t r = t->rows; r < ds::kRowsMax; ++r) p->blk_begin[r + 1] = p->blk_begin[r];
  return DS_OK;
}

}  // namespace

extern "C" {

size_t ds_rows_indexer_mq_scores_elems(const ds_indexer_rows *rows, uint32_t query_len) {
  MqPlan p;
  if (check_mq(rows, query_len, &p) != DS_OK) return 0;
  return static_cast<size_t>(uint64_t(p.rows) * query_len * p.max_kv);
}

ds_status ds_rows_indexer_score_mq(const ds_indexer_rows *rows, uint32_t query_len, const void *q, size_t q_elems,
                                   const float *weights, size_t weights_elems, float *scores, size_t scores_elems,
                                   void *stream) {
  MqPlan p;
  DS_TRY(check_mq(rows, query_len, &p));
  DS_TRY(need(q, "indexer q"));
  DS_TRY(need(weights, "indexer weights"));
  DS_TRY(need(scores, "indexer scores"));
  for (uint32_t r = 0; r < p.rows; ++r) {
    if (!rows->keys[r]) return fail("indexer row %u: keys must not be null", r);
    DS_TRY(cap(rows->keys_elems[r], uint64_t(rows->kv_len[r]) * DS_INDEXER_DIM, "indexer kv", "elements"));
  }
  DS_TRY(cap(q_elems, p.q_rows * DS_HEADS * DS_INDEXER_DIM, "indexer q", "elements"));
  DS_TRY(cap(weights_elems, p.q_rows * DS_HEADS, "indexer weights", "elements"));
  DS_TRY(cap(scores_elems, uint64_t(p.rows) * query_len * p.max_kv, "indexer scores", "elements"));
  DS_TRY(check_device());

  ds::IndexerMqArgs a{};
  a.q = static_cast<const uint16_t *>(q);
  a.w = weights;
  a.scores = scores;
  a.score_stride = p.max_kv;
  a.rows = p.rows;
  a.query_len = query_len;
  a.keys_per_block = kMqKeysPerBlock;
  for (uint32_t r = 0; r <= ds::kRowsMax; ++r) a.blk_begin[r] = p.blk_begin[r];
  for (uint32_t r = 0; r < p.rows; ++r) {
    a.keys[r] = static_cast<const uint16_t *>(rows->keys[r]);
    a.kv_len[r] = rows->kv_len[r];
    a.q_row[r] = rows->q_row[r];
    for (uint32_t t = 0; t < query_len; ++t)
      a.visible[r * ds::kMqMaxQueries + t] = std::min<uint32_t>(rows->kv_len[r], (rows->start_pos[r] + t + 1) / DS_RATIO);
  }
  uint32_t max_row_blocks = 1;
  for (uint32_t r = 0; r < p.rows; ++r) max_row_blocks = std::max(max_row_blocks, p.blk_begin[r + 1] - p.blk_begin[r]);
  const hipError_t e = ds::launch_indexer_mq(a, max_row_blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DS_OK : hip_fail(e, "multi-query indexer launch");
}

}  // extern "C"
