// A row's final top-k level and its sparse attention in one kernel.
//
// What is computed is exactly ds_rows_indexer_topk's last level followed by
// ds_rows_sparse_attn_direct on its indices (rows whose selection ended in
// an earlier pass read their indices from the output). That level is either
// the best 512 of the fused indexer's candidates in rank order, checked
// against the waves' floors, with the reselection from scores when a floor
// could hide a ranking key, or, for rows whose visible scores all fit one
// selection chunk, the best 512 of the scores themselves. Sources: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
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
// The attention's combine kernel follows. (Combining in this kernel, by the
// last workgroup of each (row, head group) to finish, with the chunk results
// passed through agent-scope stores and loads and an arrival counter, was
// measured slower: 26.6 us for final level + attention + combine against
// about 18 us with the separate kernel, at 8 rows x 32768 keys.)
#include "attn_chunk.hpp"
#include "topk_select.hpp"

namespace ds {

// The row's arguments of both parts (its final top-k level and its attention
// chunk, direct variant) read in one batch of scalar loads at entry, waited
// for once; rows and chunks are read in the same batch.
__device__ __forceinline__ void topk_attn_rows(const TopkLevelArgs &t, const AttnArgs &a, uint32_t r, uint32_t &rows,
                                               uint32_t &chunks, LevelRow &lr, AttnRow &ar, int32_t *&out) {
  uint64_t in = reinterpret_cast<uint64_t>(t.in), in_base = t.in_base[r];
  uint64_t sc = reinterpret_cast<uint64_t>(t.scores), stride = t.score_stride;
  uint64_t fl = reinterpret_cast<uint64_t>(t.floors);
  uint32_t floor_begin = t.floor_begin[r], count = t.count[r], fc = t.floor_count[r], fb = t.fallback_count[r];
  uint32_t off = static_cast<uint32_t>(t.offset[r]), fmask = t.final_mask, cmask = t.check_mask;
  uint64_t ibits = reinterpret_cast<uint64_t>(t.indices);
  uint32_t out_off = t.out_offset[r];
  uint64_t kv = reinterpret_cast<uint64_t>(a.kv[r]), q = reinterpret_cast<uint64_t>(a.q);
  uint64_t sinks = reinterpret_cast<uint64_t>(a.sinks);
  uint64_t stats = reinterpret_cast<uint64_t>(a.stats), stat_base = a.stat_base[r];
  uint64_t opart = reinterpret_cast<uint64_t>(a.opart), part_base = a.part_base[r];
  uint32_t q_row = a.q_row[r], width = a.width[r], kv_len = a.kv_len[r], scale = __float_as_uint(a.scale);
  rows = a.rows;
  chunks = a.chunks[r];
  asm volatile("" : "+s"(in), "+s"(in_base), "+s"(sc), "+s"(stride), "+s"(fl), "+s"(floor_begin), "+s"(count),
               "+s"(fc), "+s"(fb), "+s"(off), "+s"(fmask), "+s"(cmask), "+s"(kv), "+s"(q), "+s"(sinks), "+s"(stats),
               "+s"(stat_base), "+s"(opart), "+s"(part_base), "+s"(q_row), "+s"(width), "+s"(kv_len), "+s"(scale),
               "+s"(rows), "+s"(chunks), "+s"(ibits), "+s"(out_off));
  out = global_ptr<int32_t>(ibits) + out_off;
  lr.in = global_ptr<const uint64_t>(in) + in_base;
  lr.scores = global_ptr<const float>(sc) + r * stride;
  lr.floors = global_ptr<const uint64_t>(fl) + floor_begin;
  lr.out = nullptr;   // a final level writes indices, not lists
  lr.count = count;
  lr.floor_count = fc;
  lr.fallback_count = fb;
  lr.offset = static_cast<int32_t>(off);
  lr.final_level = ((fmask >> r) & 1u) != 0;
  lr.check = lr.final_level && ((cmask >> r) & 1u) != 0;
  ar.rows = global_ptr<const uint16_t>(kv);
  ar.mask = nullptr;   // direct variant
  ar.invalid = nullptr;
  ar.q = global_ptr<const uint16_t>(q) + static_cast<uint64_t>(q_row) * kHeads * kDim;
  ar.sinks = global_ptr<const float>(sinks);
  ar.stats = global_ptr<float4>(stats) + stat_base;
  ar.opart = global_ptr<float>(opart) + part_base;
  ar.width = width;
  ar.kv_len = kv_len;
  ar.scale = __uint_as_float(scale);
}

// The leading arguments arrive in scalar registers (kernel-argument
// preloading): the level's input lists and the fused indexer's floors, with
// the room per row of each (row r's at r * room; a list room of 0: the lists
// are not in that layout). With them the row's candidates and floors are
// loaded first, before the other arguments are read.
template <bool kFromScores, int kPer>
__global__ __launch_bounds__(kTopkThreads) void topk_attn_kernel(const uint64_t *lists, const uint64_t *floors,
                                                                 uint32_t list_room, uint32_t floor_room,
                                                                 TopkLevelArgs t, AttnArgs a) {
  __shared__ union Shared {
    TopkShared sel;
    AttnChunkShared att;
  } u;
  __shared__ int32_t slot_index[kAttnChunk];

  // Grid (x, row), as the attention's phase 1.
  const uint32_t r = blockIdx.y;
  const uint32_t tid = threadIdx.x;
  const bool have_pre = !kFromScores && list_room != 0;   // uniform
  const bool have_pre_floor = !kFromScores && floor_room != 0;
  uint64_t pre_keys[kPer] = {};
  uint64_t pre_floor = 0;
  if constexpr (!kFromScores) {
    // Unconditional loads (both pointers are valid for a level over lists;
    // a room of 0 reads entry 0, unused), so that nothing waits for them
    // before the selection does.
    const uint64_t *row = lists + static_cast<uint64_t>(r) * list_room;
    const uint32_t last = list_room > 0 ? list_room - 1 : 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) pre_keys[e] = row[min(tid + kTopkThreads * e, last)];
    const uint32_t flast = floor_room > 0 ? floor_room - 1 : 0;
    pre_floor = floors[static_cast<uint64_t>(r) * floor_room + min(tid, flast)];
  }
  uint32_t c, hg;
  attn_block(blockIdx.x, c, hg);
  uint32_t rows, chunks;
  LevelRow lr;
  AttnRow ar;
  int32_t *out;   // the row's index output
  topk_attn_rows(t, a, r, rows, chunks, lr, ar, out);
  if (r >= rows || c >= chunks) return;   // uniform
  const uint32_t lo = c * kAttnChunk;
  // Head group 0 writes the index output: each chunk its own 64 slots, the
  // last chunk also every slot past the row's width.
  const uint32_t out_end = c + 1 == chunks ? static_cast<uint32_t>(kTopK) : lo + kAttnChunk;
  if (lr.final_level) {   // uniform
    select_level<kFromScores, kPer>(
        u.sel, lr, 0,
        [&](uint32_t pos, int32_t index) {
          if (pos - lo < static_cast<uint32_t>(kAttnChunk)) slot_index[pos - lo] = index;   // pos in [lo, lo + 64)
          if (hg == 0 && pos >= lo && pos < out_end) out[pos] = index;
        },
        have_pre, pre_keys, have_pre_floor, pre_floor);
  } else if (threadIdx.x < static_cast<uint32_t>(kAttnChunk)) {
    // The row finished its selection in an earlier pass: its indices are in
    // the output already.
    slot_index[threadIdx.x] = out[min(lo + threadIdx.x, static_cast<uint32_t>(kTopK) - 1)];
  }
  __syncthreads();   // the chunk's indices are in place; the selection's LDS is free
  static_assert(kTopkThreads == kChunkThreads, "the attention chunk uses every thread of the workgroup");
  attn_chunk_body<true>(u.att, ar, hg, c, [&](uint32_t slot) { return slot_index[slot - lo]; });
}

hipError_t launch_topk_attn(const TopkLevelArgs &t, const AttnArgs &a, uint32_t max_chunks, hipStream_t s) {
  const dim3 blocks(kXcds * kAttnHeadGroups * ((max_chunks + kXcds - 1) / kXcds), a.rows);
  // A level without floors passes its lists in their place (a valid address
  // for the kernel's unconditional floor load) and a floor room of 0.
  const uint64_t *fl = t.floors != nullptr ? t.floors : t.in;
  const uint32_t froom = t.floors != nullptr ? t.floor_room : 0;
  if (t.from_scores) {
    // The scores of every row fit one chunk of 4, 8 or 16 per thread.
    if (t.per_thread == 4)
      hipLaunchKernelGGL((topk_attn_kernel<true, 4>), dim3(blocks), dim3(kTopkThreads), 0, s, t.in, fl, t.list_room, froom, t, a);
    else if (t.per_thread == 8)
      hipLaunchKernelGGL((topk_attn_kernel<true, 8>), dim3(blocks), dim3(kTopkThreads), 0, s, t.in, fl, t.list_room, froom, t, a);
    else
      hipLaunchKernelGGL((topk_attn_kernel<true, 16>), dim3(blocks), dim3(kTopkThreads), 0, s, t.in, fl, t.list_room, froom, t, a);
  } else if (t.per_thread == 4)
    hipLaunchKernelGGL((topk_attn_kernel<false, 4>), dim3(blocks), dim3(kTopkThreads), 0, s, t.in, fl, t.list_room, froom, t, a);
  else if (t.per_thread == 16)
    hipLaunchKernelGGL((topk_attn_kernel<false, 16>), dim3(blocks), dim3(kTopkThreads), 0, s, t.in, fl, t.list_room, froom, t, a);
  else
    hipLaunchKernelGGL((topk_attn_kernel<false, kTopkPerThreadLater>), dim3(blocks), dim3(kTopkThreads), 0, s, t.in, fl, t.list_room, froom, t, a);
  return hipGetLastError();
}

}  // namespace ds
