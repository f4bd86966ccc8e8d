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

// Cross-lane steps by DPP (row = 16 lanes). update_dpp(old, v, ...) gives
// each lane the moved value, or `old` where the source lies outside the row
// or the lane's row is masked off.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 to rows 2 and 3
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), kCtrl, kRowMask, 0xF, false));
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<kCtrl>(0u, __float_as_uint(v)));
}

// Inclusive prefix over the 64 lanes of a wave in lane order (sum or max of
// unsigned values): doubling steps inside each row, then the row totals
// carried into the rows above.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  x += dpp_u32<kDppRowShr1>(0u, x);
  x += dpp_u32<kDppRowShr2>(0u, x);
  x += dpp_u32<kDppRowShr4>(0u, x);
  x += dpp_u32<kDppRowShr8>(0u, x);
  x += dpp_u32<kDppRowBcast15, 0xA>(0u, x);
  x += dpp_u32<kDppRowBcast31, 0xC>(0u, x);
  return x;
}
__device__ __forceinline__ uint32_t wave_prefix_max(uint32_t x) {
  x = max(x, dpp_u32<kDppRowShr1>(0u, x));
  x = max(x, dpp_u32<kDppRowShr2>(0u, x));
  x = max(x, dpp_u32<kDppRowShr4>(0u, x));
  x = max(x, dpp_u32<kDppRowShr8>(0u, x));
  x = max(x, dpp_u32<kDppRowBcast15, 0xA>(0u, x));
  x = max(x, dpp_u32<kDppRowBcast31, 0xC>(0u, x));
  return x;
}

// Whole-wave reductions, the result in every lane: inside each row by
// rotations and pair swaps, then across row pairs (v_permlane16_swap) and
// wave halves (v_permlane32_swap). Each step combines a lane with a partner
// holding the same two operands in the other order, so every lane ends with
// the same bits (also for floating point).
// (Every lane has a source lane in these rotations and swaps, so the moves'
// `old` operand is never used; passing 0 rather than x lets the compiler fold
// each move into its operation, one DPP instruction per step instead of a
// copy, a wait state, a move and the operation.)
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, Op op) {
  x = op(x, dpp_u32<kDppRowRor8>(0u, x));
  x = op(x, dpp_u32<kDppRowRor4>(0u, x));
  x = op(x, dpp_u32<kDppQuadSwap2>(0u, x));
  x = op(x, dpp_u32<kDppQuadSwap1>(0u, x));
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r[0], r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(h[0], h[1]);
}
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t p, uint32_t q) { return p + q; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t p, uint32_t q) { return min(p, q); });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return wave_reduce_u32(x, [](uint32_t p, uint32_t q) { return max(p, q); });
}

// Reductions over the 32 lanes of a wave half (lanes 0..31 or 32..63), the
// result in every lane of the half (same scheme, without the last step).
__device__ __forceinline__ float half_sum(float v) {
  v += dpp_f32<kDppRowRor8>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppQuadSwap2>(v);
  v += dpp_f32<kDppQuadSwap1>(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Whether any lane of this lane's 32-lane half has the flag set.
__device__ __forceinline__ bool half_any(bool f) {
  const uint64_t m = __ballot(f);
  return ((m >> (__lane_id() & 32u)) & 0xFFFFFFFFull) != 0;
}

// Whole-wave float reductions, the result in every lane: the half-wave
// reduction, then the two halves (v_permlane32_swap), so that every lane ends
// with the same bits.
__device__ __forceinline__ float wave_sum_f(float v) {
  v = half_sum(v);
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// max(x, 0) with maxNum's treatment of a NaN input (the result is 0) in one
// instruction: v_med3_f32(x, 0, +inf) is the median, and for a quiet NaN
// operand the hardware returns the smallest of the three, 0. (fmaxf costs a
// second instruction that quiets signalling NaNs first; the values clamped
// here are MFMA results, never signalling.) A -0 result may come back as
// either zero, which no use here can tell apart.
// `inf` is +inf held in a register the compiler cannot see into (see
// opaque_inf), so that it emits the med3 rather than folding it back into a
// max with the quieting instruction.
__device__ __forceinline__ float opaque_inf() {
  float inf = __builtin_inff();
  asm volatile("" : "+v"(inf));
  return inf;
}
__device__ __forceinline__ float relu_num(float x, float inf) { return __builtin_amdgcn_fmed3f(x, 0.0f, inf); }

// Maxima of values that are never NaN (finite or infinite), over the 32
// lanes of a wave half and over the whole wave, in every lane: the scheme of
// half_sum / wave_sum_f with max(a, b) as the median of a, b and +inf, one
// instruction per step (fmaxf adds a NaN-quieting instruction to each).
// The maximum is exact, so every lane ends with the same bits. (A med3
// cannot take a DPP operand, so the lane moves are plain DPP moves: every
// lane has a source in these patterns.)
template <int kCtrl>
__device__ __forceinline__ float dpp_mov_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float half_max(float v) {
  const float inf = opaque_inf();
  v = __builtin_amdgcn_fmed3f(v, dpp_mov_f32<kDppRowRor8>(v), inf);
  v = __builtin_amdgcn_fmed3f(v, dpp_mov_f32<kDppRowRor4>(v), inf);
  v = __builtin_amdgcn_fmed3f(v, dpp_mov_f32<kDppQuadSwap2>(v), inf);
  v = __builtin_amdgcn_fmed3f(v, dpp_mov_f32<kDppQuadSwap1>(v), inf);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_amdgcn_fmed3f(__uint_as_float(r[0]), __uint_as_float(r[1]), inf);
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = half_max(v);
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_amdgcn_fmed3f(__uint_as_float(h[0]), __uint_as_float(h[1]), opaque_inf());
}

// A device pointer handed over as its integer bits (to pass it through an
// empty asm statement), rebuilt as a global-memory pointer so that accesses
// through it stay global (not flat) loads and stores.
template <class T>
__device__ __forceinline__ T *global_ptr(uint64_t bits) {
  return (T *)((__attribute__((address_space(1))) T *)bits);
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
