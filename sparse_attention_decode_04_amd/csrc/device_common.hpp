// Device-side helpers shared by the gfx950 kernels: vector types, bf16 bit
// handling and the MFMA operand conventions used throughout.
//
// MFMA lane layouts relied on (wave64, gfx950):
//   v_mfma_f32_16x16x32_bf16: A lane l holds row l%16, k = 8*(l/16)..+7;
//     B lane l holds column l%16, same k; D lane l holds column l%16,
//     rows 4*(l/16) + i for i = 0..3.
//   v_mfma_f32_32x32x16_bf16: A lane l holds row l%32, k = 8*(l/32)..+7;
//     B lane l holds column l%32, same k; D lane l holds column l%32,
//     rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
// Only the row/column placement matters for correctness: a contraction may
// assign real feature indices to k positions in any order as long as A and B
// agree, which the kernels use to give every lane contiguous 16-byte loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ds {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 load16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void store16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }

// bf16 bit pattern of a finite-or-not value: exponent all ones means
// infinity or NaN.
__device__ __forceinline__ bool bf16_bits_nonfinite(uint32_t b16) {
  return (b16 & 0x7F80u) == 0x7F80u;
}

constexpr uint16_t kBf16NegInf = 0xFF80;
constexpr uint16_t kBf16NaN = 0x7FC0;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Lane rows of 16 (rows 0..3 of the wave). With x and y per lane:
// swap_rows16_sum returns, in even rows, x(row) + x(row + 1) and in odd rows
// y(row - 1) + y(row) (v_permlane16_swap exchanges the odd rows of its first
// operand with the even rows of its second).
__device__ __forceinline__ float swap_rows16_sum(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Halves of 32 lanes: returns, in the low half, x(l) + x(l + 32) and in the
// high half y(l - 32) + y(l) (v_permlane32_swap exchanges the high half of its
// first operand with the low half of its second).
__device__ __forceinline__ float swap_halves_sum(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row of a multi-row launch owning workgroup `b`: the last r with
// blk_begin[r] <= b. Entries past the last row hold the total block count.
__device__ __forceinline__ uint32_t row_of_block(const uint32_t *blk_begin, uint32_t b) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 1; i < 8; ++i) r = (b >= blk_begin[i]) ? i : r;
  return r;
}

}  // namespace ds
