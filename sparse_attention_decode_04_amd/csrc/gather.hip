// Gather of each row's selected KV rows into one contiguous bf16 operand.
//
// Source: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernel deepseek_sparse_attention_gather_rows_bf16: per slot, a -1 index is
// a sentinel (zero row, mask -inf), an index outside [0, kv_len) is bad (zero
// row, row invalid), otherwise the KV row is copied bit for bit with
// non-finite elements replaced by zero (and the row marked invalid).
//
// Differences from the pages' kernel (one thread per element, a relaxed
// atomic store into a caller-zeroed per-row flag): one wave moves one
// 1 KiB row as 64 lanes x 16 bytes, eight rows in flight per wave, with the
// wave's eight indices read by eight lanes and broadcast; and the "row
// invalid" state is carried per slot in the mask as NaN, written with a plain
// store by the wave that saw it. The mask therefore needs no zeroed workspace
// and no atomics; the attention call treats any NaN mask entry of a row as
// the row's invalid flag.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(GatherArgs a) {
  // Grid: (blocks of the widest row, rows); row r is blockIdx.y, so its
  // arguments are read in one batch of scalar loads, waited for once.
  // Blocks past the row's width end at once.
  const uint32_t r = blockIdx.y;
  uint32_t width = a.width[r], n = a.kv_len[r], ioff = a.index_offset[r];
  uint64_t kvb = reinterpret_cast<uint64_t>(a.kv[r]), ib = reinterpret_cast<uint64_t>(a.indices);
  uint64_t gb = reinterpret_cast<uint64_t>(a.gathered), mb = reinterpret_cast<uint64_t>(a.mask), sbase = a.slot_base[r];
  asm volatile("" : "+s"(width), "+s"(n), "+s"(ioff), "+s"(kvb), "+s"(ib), "+s"(gb), "+s"(mb), "+s"(sbase));
  if (blockIdx.x * kGatherSlotsPerBlock >= width) return;   // uniform
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t slot0 = blockIdx.x * kGatherSlotsPerBlock + wave * kGatherSlotsPerWave;
  const uint16_t *__restrict__ kv = global_ptr<const uint16_t>(kvb);
  const int32_t *__restrict__ idx = global_ptr<const int32_t>(ib) + ioff;
  uint16_t *const gathered = global_ptr<uint16_t>(gb);
  uint16_t *const mask = global_ptr<uint16_t>(mb);

  // Loads are unconditional (clamped to valid slots / KV row 0) and masked
  // afterwards, so all eight rows are in flight together.
  const uint32_t my_slot = min(slot0 + (lane % kGatherSlotsPerWave), width - 1);
  const int32_t my_raw = idx[my_slot];
  const int32_t my = (slot0 + (lane % kGatherSlotsPerWave) < width) ? my_raw : -1;
  int32_t sel[kGatherSlotsPerWave];
  u32x4 v[kGatherSlotsPerWave];
#pragma unroll
  for (int s = 0; s < kGatherSlotsPerWave; ++s) {
    sel[s] = __shfl(my, s);
    const bool ok = sel[s] >= 0 && static_cast<uint32_t>(sel[s]) < n;
    v[s] = load16(kv + static_cast<uint64_t>(ok ? sel[s] : 0) * kDim + 8 * lane);
  }
#pragma unroll
  for (int s = 0; s < kGatherSlotsPerWave; ++s) {
    const bool ok = sel[s] >= 0 && static_cast<uint32_t>(sel[s]) < n;
    if (!ok) v[s] = u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int s = 0; s < kGatherSlotsPerWave; ++s) {
    const uint32_t slot = slot0 + s;
    if (slot >= width) break;
    const bool sentinel = sel[s] == -1;
    const bool index_bad = sel[s] < -1 || (sel[s] >= 0 && static_cast<uint32_t>(sel[s]) >= n);
    bool value_bad = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t d = v[s][k];
      if (bf16_bits_nonfinite(d & 0xFFFFu)) { d &= 0xFFFF0000u; value_bad = true; }
      if (bf16_bits_nonfinite(d >> 16)) { d &= 0x0000FFFFu; value_bad = true; }
      v[s][k] = d;
    }
    const uint64_t out_slot = sbase + slot;
    store16(gathered + out_slot * kDim + 8 * lane, v[s]);
    const bool any_bad = __ballot(value_bad) != 0;
    if (lane == 0)
      mask[out_slot] = sentinel ? kBf16NegInf : ((index_bad || any_bad) ? kBf16NaN : uint16_t(0));
  }
}

hipError_t launch_gather(const GatherArgs &a, uint32_t max_row_blocks, hipStream_t s) {
  hipLaunchKernelGGL(gather_kernel, dim3(max_row_blocks, a.rows), dim3(kGatherThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
