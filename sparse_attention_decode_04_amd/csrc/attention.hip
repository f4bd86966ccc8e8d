// Sparse MQA attention over the gathered rows (keys = values) with a learned
// per-head sink, bf16 MFMA with f32 accumulation on gfx950.
//
// What is computed (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernels deepseek_sparse_attention_score_rows_bf16 and
// deepseek_sparse_attention_reduce_rows_bf16; keys = values and one sink
// vector for every row per "mlx-native 0.21.0 src/ops/deepseek_rows.rs",
// dispatch_deepseek_sparse_attention_flash_rows):
//   l[h,t] = scale * q[h] . G[t]                   (live slots only)
//   m = max(sink[h], max_t l), Z = e^(sink-m) + sum_t e^(l-m)
//   out[h] = sum_t e^(l-m)/Z * G[t]
// with the pages' fail-closed rule: a row with a bad slot (NaN mask), a head
// whose sink or any live logit is not finite, or a denominator outside
// (0, inf) is written as zeros; other non-finite outputs are zeroed.
//
// Two launches (the pages instead re-read the selected KV per (row, head) in
// a reduce kernel, or run a flash kernel per distinct width):
//   phase 1, per (row, 32-slot chunk): all 64 heads' logits by MFMA
//     32x32x16 (M = 32 heads, N = 32 slots, K = 16 features); per head the
//     chunk max m_c, p~ = exp(l - m_c) and s_c = sum p~, plus a bad flag.
//   phase 2, per (row, 32-feature chunk): m and Z from the chunk statistics
//     and the sink, then out = sum_t (p~ * e^(m_c - m) / Z) * G[t] by MFMA
//     32x32x16 with M = 32 heads, N = 32 features, K = 16 slots. The weights
//     enter as a bf16 hi + lo pair (hi = bf16(x), lo = bf16(x - hi)), so the
//     product carries ~16 significant bits of each weight; G is exact bf16.
//     MFMA operands must hold 8 consecutive K elements per lane, so the
//     slot-major KV slice is transposed into LDS (feature-major) first.
// All splits depend only on the row's own width, so rows are independent
// bit for bit.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// Mask entry states written by the gather: -inf sentinel, NaN bad, else live.
enum : uint32_t { kLive = 0, kSkip = 1, kBad = 2 };

__device__ __forceinline__ uint32_t mask_state(uint16_t m) {
  if (m == kBf16NegInf) return kSkip;
  if ((m & 0x7FFFu) > 0x7F80u) return kBad;
  return kLive;
}

constexpr int kP1Threads = 128;   // 2 waves: heads 0-31, 32-63
constexpr int kP2Threads = 128;   // 2 waves: heads 0-31, 32-63
constexpr int kLStride = kAttnChunk + 1;
constexpr int kGtStride = kAttnSuper + 8;   // bf16 elements per LDS feature row

__global__ __launch_bounds__(kP1Threads) void attn_logits_kernel(AttnArgs a) {
  __shared__ float L[kHeads * kLStride];
  __shared__ uint32_t state[kAttnChunk];

  const uint32_t r = row_of_block(a.blk_begin, blockIdx.x);
  const uint32_t c = blockIdx.x - a.blk_begin[r];
  const uint32_t width = a.width[r];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t hh = tid >> 6;
  const uint32_t col = lane & 31;
  const uint32_t g = lane >> 5;
  const uint64_t slot_base = a.slot_base[r];

  if (tid < kAttnChunk) {
    const uint32_t slot = c * kAttnChunk + tid;
    state[tid] = slot < width ? mask_state(a.mask[slot_base + slot]) : kSkip;
  }

  // A: query row 32*hh + col; B: gathered slot c*32 + col (clamped in the
  // tail). Lane group g covers features [256g, 256g + 256); step s takes
  // features 256g + 8s .. +8 for both operands.
  const uint16_t *qrow = a.q + (static_cast<uint64_t>(a.q_row[r]) * kHeads + 32 * hh + col) * kDim + 256 * g;
  const uint32_t slot = min(c * kAttnChunk + col, width - 1);
  const uint16_t *grow = a.gathered + (slot_base + slot) * kDim + 256 * g;

  f32x16 acc = {};
  u32x4 qa[4], gb[4], qn[4], gn[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) { qa[s] = load16(qrow + 8 * s); gb[s] = load16(grow + 8 * s); }
#pragma unroll
  for (int s0 = 0; s0 < 32; s0 += 4) {
    if (s0 + 4 < 32) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        qn[s] = load16(qrow + 8 * (s0 + 4 + s));
        gn[s] = load16(grow + 8 * (s0 + 4 + s));
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma32(as_bf16x8(qa[s]), as_bf16x8(gb[s]), acc);
    if (s0 + 4 < 32) {
#pragma unroll
      for (int s = 0; s < 4; ++s) { qa[s] = qn[s]; gb[s] = gn[s]; }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t head = 32 * hh + 8 * (i / 4) + 4 * g + (i % 4);
    L[head * kLStride + col] = acc[i] * a.scale;
  }
  __syncthreads();

  // Thread t: head t/2, slots 16*(t%2) .. +16 of the chunk.
  const uint32_t head = tid >> 1;
  const uint32_t half = tid & 1;
  float lv[16];
  bool bad = false;
  float mx = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t st = state[16 * half + j];
    lv[j] = L[head * kLStride + 16 * half + j];
    const bool live = st == kLive;
    bad |= (st == kBad) || (live && !__builtin_isfinite(lv[j]));
    if (live && __builtin_isfinite(lv[j])) mx = fmaxf(mx, lv[j]);
  }
  const float mc = fmaxf(mx, __shfl_xor(mx, 1));
  bad = bad || (__shfl_xor(static_cast<int>(bad), 1) != 0);
  float ssum = 0.0f;
  f32x4 pv[4];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const bool live = state[16 * half + j] == kLive && __builtin_isfinite(lv[j]);
    const float p = live ? expf(lv[j] - mc) : 0.0f;
    pv[j / 4][j % 4] = p;
    ssum += p;
  }
  const float sc = ssum + __shfl_xor(ssum, 1);
  const uint32_t w32 = a.chunks[r] * kAttnChunk;
  float *prow = a.p + a.p_base[r] + static_cast<uint64_t>(head) * w32 + c * kAttnChunk + 16 * half;
#pragma unroll
  for (int k = 0; k < 4; ++k) *reinterpret_cast<f32x4 *>(prow + 4 * k) = pv[k];
  if (half == 0)
    a.stats[a.stat_base[r] + static_cast<uint64_t>(head) * a.chunks[r] + c] =
        make_float4(mc, sc, bad ? 1.0f : 0.0f, 0.0f);
}

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__global__ __launch_bounds__(kP2Threads) void attn_reduce_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t gt[kAttnDimChunk * kGtStride];
  __shared__ float s_m[kHeads], s_invz[kHeads];
  __shared__ uint32_t s_bad[kHeads];

  constexpr uint32_t kDimChunks = kDim / kAttnDimChunk;
  const uint32_t r = blockIdx.x / kDimChunks;
  const uint32_t dc = blockIdx.x % kDimChunks;
  const uint32_t width = a.width[r];
  const uint32_t nch = a.chunks[r];
  const uint32_t w32 = nch * kAttnChunk;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t hh = tid >> 6;
  const uint32_t col = lane & 31;
  const uint32_t g = lane >> 5;
  const float4 *stats = a.stats + a.stat_base[r];

  // Softmax statistics per head from the chunk maxima/sums and the sink.
  if (tid < kHeads) {
    const float sink = a.sinks[tid];
    bool bad = !__builtin_isfinite(sink);
    float m = bad ? 0.0f : sink;
    for (uint32_t c = 0; c < nch; ++c) {
      const float4 st = stats[tid * nch + c];
      bad |= st.z != 0.0f;
      if (st.y > 0.0f) m = fmaxf(m, st.x);
    }
    float z = bad ? 1.0f : expf(sink - m);
    for (uint32_t c = 0; c < nch; ++c) {
      const float4 st = stats[tid * nch + c];
      if (st.y > 0.0f) z += st.y * expf(st.x - m);
    }
    bad |= !(z > 0.0f && __builtin_isfinite(z));
    s_m[tid] = m;
    s_invz[tid] = bad ? 0.0f : 1.0f / z;
    s_bad[tid] = bad ? 1u : 0u;
  }

  const uint32_t ahead = 32 * hh + col;                 // A row of this lane
  const float *prow = a.p + a.p_base[r] + static_cast<uint64_t>(ahead) * w32;
  const float4 *srow = stats + static_cast<uint64_t>(ahead) * nch;
  const uint16_t *gbase = a.gathered + a.slot_base[r] * kDim + dc * kAttnDimChunk;

  f32x16 acc = {};
  for (uint32_t s0 = 0; s0 < width; s0 += kAttnSuper) {
    const uint32_t span = min(width - s0, static_cast<uint32_t>(kAttnSuper));
    __syncthreads();   // previous span's LDS reads are done (and stats above)
    // Stage G[s0 .. s0+512, features dc*32 .. +32] feature-major: each thread
    // moves 8x8 blocks (8 slots x 8 features), transposing in registers.
    for (uint32_t b = tid; b < (kAttnSuper / 8) * (kAttnDimChunk / 8); b += kP2Threads) {
      const uint32_t sb = b / (kAttnDimChunk / 8);
      const uint32_t fb = b % (kAttnDimChunk / 8);
      u16x8 rows[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sl = 8 * sb + i;
        rows[i] = sl < span ? __builtin_bit_cast(u16x8, load16(gbase + static_cast<uint64_t>(s0 + sl) * kDim + 8 * fb))
                            : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u16x8 colv;
#pragma unroll
        for (int i = 0; i < 8; ++i) colv[i] = rows[i][j];
        *reinterpret_cast<u16x8 *>(&gt[(8 * fb + j) * kGtStride + 8 * sb]) = colv;
      }
    }
    __syncthreads();

    const float m = s_m[ahead];
    const float invz = s_invz[ahead];
    const uint32_t steps = (span + 15) / 16;
    for (uint32_t k = 0; k < steps; ++k) {
      const uint32_t sl = 16 * k + 8 * g;               // first of this lane's 8 slots
      const uint32_t chunk = (s0 + sl) / kAttnChunk;
      const float mc = srow[chunk].x;
      const float f = (mc == -__builtin_inff()) ? 0.0f : expf(mc - m) * invz;
      const f32x4 p0 = *reinterpret_cast<const f32x4 *>(prow + s0 + sl);
      const f32x4 p1 = *reinterpret_cast<const f32x4 *>(prow + s0 + sl + 4);
      u16x8 hi, lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = (i < 4 ? p0[i] : p1[i - 4]) * f;
        hi[i] = bf16_rne_bits(x);
        lo[i] = bf16_rne_bits(x - bf16_bits_to_float(hi[i]));
      }
      const u16x8 bv = *reinterpret_cast<const u16x8 *>(&gt[col * kGtStride + sl]);
      acc = mfma32(__builtin_bit_cast(bf16x8, hi), __builtin_bit_cast(bf16x8, bv), acc);
      acc = mfma32(__builtin_bit_cast(bf16x8, lo), __builtin_bit_cast(bf16x8, bv), acc);
    }
  }

  const uint64_t obase = static_cast<uint64_t>(a.q_row[r]) * kHeads * kDim + dc * kAttnDimChunk + col;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t head = 32 * hh + 8 * (i / 4) + 4 * g + (i % 4);
    const float v = acc[i];
    a.out[obase + static_cast<uint64_t>(head) * kDim] = (s_bad[head] == 0 && __builtin_isfinite(v)) ? v : 0.0f;
  }
}

hipError_t launch_attn_logits(const AttnArgs &a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(attn_logits_kernel, dim3(blocks), dim3(kP1Threads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_reduce(const AttnArgs &a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(attn_reduce_kernel, dim3(blocks), dim3(kP2Threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
