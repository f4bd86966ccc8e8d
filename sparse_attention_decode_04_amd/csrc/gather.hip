// Gather of each row's selected KV rows into one contiguous bf16 operand.
//
// Source: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernel deepseek_sparse_attention_gather_rows_bf16: per slot, a -1 index is
// a sentinel (zero row, mask -inf), an index outside [0, kv_len) is bad (zero
// row, mask 0, row invalid), otherwise the KV row is copied bit for bit with
// non-finite elements replaced by zero (and the row marked invalid).
//
// Differences from the pages' kernel (one thread per element; a relaxed
// atomic store into a per-row flag the caller has cleared): one wave moves
// one 1 KiB row as 64 lanes x 16 bytes, eight rows in flight per wave, with
// the wave's eight indices read by eight lanes and broadcast; the per-row
// flag is cleared by a first one-workgroup kernel of the same call (so the
// caller need not), and each wave that saw a bad slot sets it with one atomic
// OR.
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
  uint64_t vb = reinterpret_cast<uint64_t>(a.invalid);
  asm volatile("" : "+s"(width), "+s"(n), "+s"(ioff), "+s"(kvb), "+s"(ib), "+s"(gb), "+s"(mb), "+s"(sbase), "+s"(vb));
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
  bool row_bad = false;   // wave-uniform
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
    row_bad |= index_bad || __ballot(value_bad) != 0;
    if (lane == 0) mask[out_slot] = sentinel ? kBf16NegInf : uint16_t(0);
  }
  if (row_bad && lane == 0) atomicOr(global_ptr<uint32_t>(vb) + r, 1u);
}

// invalid[0 .. rows) = 0, ahead of the gather in the same stream.
__global__ __launch_bounds__(64) void clear_flags_kernel(uint32_t *flags, uint32_t n) {
  if (threadIdx.x < n) flags[threadIdx.x] = 0;
}

hipError_t launch_gather(const GatherArgs &a, uint32_t max_row_blocks, hipStream_t s) {
  static_assert(kRowsMax <= 64, "one clearing workgroup");
  hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(64), 0, s, a.invalid, a.rows);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gather_kernel, dim3(max_row_blocks, a.rows), dim3(kGatherThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
