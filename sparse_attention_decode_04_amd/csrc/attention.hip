// Sparse MQA attention over the selected KV rows (keys = values) with a
// learned per-head sink, bf16 MFMA with f32 accumulation on gfx950.
//
// What is computed (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernels deepseek_sparse_attention_score_rows_bf16 and
// deepseek_sparse_attention_reduce_rows_bf16, and the gather semantics of
// deepseek_sparse_attention_gather_rows_bf16; keys = values and one sink
// vector for every row per "mlx-native 0.21.0 src/ops/deepseek_rows.rs",
// dispatch_deepseek_sparse_attention_flash_rows):
//   l[h,t] = scale * q[h] . G[t]                   (live slots only)
//   m = max(sink[h], max_t l), Z = e^(sink-m) + sum_t e^(l-m)
//   out[h] = sum_t e^(l-m)/Z * G[t]
// with the pages' fail-closed rule: a row with a bad slot (bad index or a
// non-finite KV element), a head whose sink or any live logit is not finite,
// or a denominator outside (0, inf) is written as zeros; other non-finite
// outputs are zeroed.
//
// Two launches. The selected rows G[t] come either from the gathered operand
// and its mask (after ds_rows_gather) or, in the direct variant, straight from
// each row's KV through the indices (the gather fused in).
//   phase 1, per (row, 32-slot chunk), 8 waves: logits on MFMA 32x32x16
//     (M = 32 heads, N = 32 slots, K = 16 features); waves split heads in two
//     and features in four, issue all their loads at once, and sum the four
//     partial tiles in LDS in a fixed order. Per head: the chunk max m_c,
//     p~ = exp(l - m_c) stored as a bf16 pair (hi = bf16(p~),
//     lo = bf16(p~ - hi): ~16 significant bits) and s_c = sum p~. The chunk's
//     rows are also written feature-major (G^T) for phase 2.
//   phase 2, per (row, 32-feature chunk), 8 waves: m and Z per head from the
//     chunk statistics and the sink, a factor e^(m_c - m)/Z per (chunk, head)
//     in LDS, then out = sum_c factor_c * (p~ . G)_c with the inner products
//     on MFMA 32x32x16 (M = 32 heads, N = 32 features, K = 16 slots) into a
//     per-chunk accumulator. Waves split heads in two and slots in four; the
//     four partial outputs are summed in LDS in a fixed order. Both MFMA
//     operands need 8 consecutive slots per lane, which is why phase 1 stores
//     p~ slot-major per head and G feature-major.
// All splits depend only on the row's own width, so rows are independent
// bit for bit.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

// Slot states: -inf mask / -1 index = sentinel, NaN mask / bad index = bad.
enum : uint32_t { kLive = 0, kSkip = 1, kBad = 2 };

__device__ __forceinline__ uint32_t mask_state(uint16_t m) {
  if (m == kBf16NegInf) return kSkip;
  if ((m & 0x7FFFu) > 0x7F80u) return kBad;
  return kLive;
}

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ bool any_nonfinite(u32x4 v) {
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 4; ++k) bad |= bf16_bits_nonfinite(v[k] & 0xFFFFu) || bf16_bits_nonfinite(v[k] >> 16);
  return bad;
}

constexpr int kAttnThreads = 512;   // 8 waves: 2 head halves x 4 K quarters
constexpr int kRedStride = 33;      // padded row of a 32-wide f32 tile in LDS
constexpr int kChunkStride = kDim + 8;   // bf16 per LDS slot row (phase 1 G^T staging)
constexpr int kChunksPerSuper = kAttnSuper / kAttnChunk;     // 16

// ---------------------------------------------------------------- phase 1
template <bool kDirect>
__global__ __launch_bounds__(kAttnThreads) void attn_logits_kernel(AttnArgs a) {
  __shared__ float red[4 * kHeads * kRedStride];
  __shared__ __attribute__((aligned(16))) uint16_t chunk_rows[kAttnChunk * kChunkStride];
  __shared__ uint32_t state[kAttnChunk];
  __shared__ uint32_t vbad[4][2][kAttnChunk];

  // Row r runs on XCD r: consecutive workgroups go to consecutive XCDs, so
  // block b = 8 c + r puts all of a row's chunks in one L2 (its query is
  // fetched from memory once per row, not once per XCD).
  const uint32_t r = blockIdx.x % kXcds;
  const uint32_t c = blockIdx.x / kXcds;
  if (r >= a.rows || c >= a.chunks[r]) return;
  const uint32_t width = a.width[r];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t hh = wave & 1;          // heads 32*hh ..
  const uint32_t kq = wave >> 1;         // features 128*kq ..
  const uint32_t col = lane & 31;
  const uint32_t g = lane >> 5;
  const uint32_t f0 = 128 * kq + 64 * g;   // this lane group's 64 features

  // The lane's slot: its state and its source row. Loads are unconditional
  // (a slot past the width reads the row's last slot, a sentinel or bad index
  // reads KV row 0) and masked afterwards, so they are all in flight at once.
  // The slot's index (or mask entry) is loaded first: the KV row load depends
  // on it, and loads complete in issue order.
  const uint32_t slot = c * kAttnChunk + col;
  const uint32_t cslot = min(slot, width - 1);
  int32_t raw_index = 0;
  uint16_t raw_mask = 0;
  if (kDirect) raw_index = a.indices[a.index_offset[r] + cslot];
  else raw_mask = a.mask[a.slot_base[r] + cslot];

  // Query fragments: they do not depend on the slot.
  const uint16_t *qrow = a.q + (static_cast<uint64_t>(a.q_row[r]) * kHeads + 32 * hh + col) * kDim + f0;
  u32x4 qa[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qa[s] = load16(qrow + 8 * s);

  uint32_t st;
  const uint16_t *src;
  if (kDirect) {
    const int32_t i = slot < width ? raw_index : -1;
    const bool ok = i >= 0 && static_cast<uint32_t>(i) < a.kv_len[r];
    st = ok ? kLive : ((slot < width && i != -1) ? kBad : kSkip);
    src = a.kv[r] + static_cast<uint64_t>(ok ? i : 0) * kDim;
  } else {
    st = slot < width ? mask_state(raw_mask) : kSkip;
    src = a.gathered + (a.slot_base[r] + cslot) * kDim;
  }
  const bool use = kDirect ? st == kLive : slot < width;
  // This thread's head (epilogue: head tid / 8) sink, stored with the chunk
  // statistics so that phase 2 gets it in the same load.
  const float sink_h = a.sinks[tid >> 3];
  u32x4 gb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) gb[s] = load16(src + f0 + 8 * s);
#pragma unroll
  for (int s = 0; s < 8; ++s)
    if (!use) gb[s] = u32x4{0, 0, 0, 0};
  if (kDirect) {
    // Gather semantics: a non-finite element makes the row invalid.
    bool nf = false;
#pragma unroll
    for (int s = 0; s < 8; ++s) nf |= any_nonfinite(gb[s]);
    if (hh == 0) vbad[kq][g][col] = nf ? 1u : 0u;
  }
  if (tid < kAttnChunk) state[tid] = st;   // wave 0, lanes 0..31: slot == tid

  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = mfma32(as_bf16x8(qa[s]), as_bf16x8(gb[s]), acc);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t head = 32 * hh + 8 * (i / 4) + 4 * g + (i % 4);
    red[(kq * kHeads + head) * kRedStride + col] = acc[i];
  }
  if (hh == 0) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<u32x4 *>(&chunk_rows[col * kChunkStride + f0 + 8 * s]) = gb[s];
  }
  __syncthreads();

  // G^T for phase 2: 8-slot x 8-feature blocks transposed in registers.
  // Slots past the width are written as zero rows.
  if (tid < (kAttnChunk / 8) * (kDim / 8)) {
    const uint32_t sb = tid % (kAttnChunk / 8);
    const uint32_t fb = tid / (kAttnChunk / 8);
    u16x8 rows[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rows[i] = *reinterpret_cast<const u16x8 *>(&chunk_rows[(8 * sb + i) * kChunkStride + 8 * fb]);
    const uint32_t w32 = a.chunks[r] * kAttnChunk;
    uint16_t *dst = a.gt + a.gt_base[r] + static_cast<uint64_t>(8 * fb) * w32 + c * kAttnChunk + 8 * sb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      u16x8 colv;
#pragma unroll
      for (int i = 0; i < 8; ++i) colv[i] = rows[i][j];
      *reinterpret_cast<u16x8 *>(dst + static_cast<uint64_t>(j) * w32) = colv;
    }
  }

  // Thread t: head t/8, slots 4*(t%8) .. +4 of the chunk.
  const uint32_t head = tid >> 3;
  const uint32_t part = tid & 7;
  float lv[4];
  uint32_t sj[4];
  bool bad = false;
  float mx = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sl = 4 * part + j;
    float v = red[(0 * kHeads + head) * kRedStride + sl];
    v += red[(1 * kHeads + head) * kRedStride + sl];
    v += red[(2 * kHeads + head) * kRedStride + sl];
    v += red[(3 * kHeads + head) * kRedStride + sl];
    lv[j] = v * a.scale;
    sj[j] = state[sl];
    if (kDirect && sj[j] == kLive &&
        (vbad[0][0][sl] | vbad[0][1][sl] | vbad[1][0][sl] | vbad[1][1][sl] |
         vbad[2][0][sl] | vbad[2][1][sl] | vbad[3][0][sl] | vbad[3][1][sl]))
      sj[j] = kBad;
    const bool live = sj[j] == kLive;
    bad |= (sj[j] == kBad) || (live && !__builtin_isfinite(lv[j]));
    if (live && __builtin_isfinite(lv[j])) mx = fmaxf(mx, lv[j]);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    const int other = __shfl_xor(static_cast<int>(bad), o);   // every lane must take part
    bad = bad || other != 0;
  }
  float ssum = 0.0f;
  u16x4 hi, lo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool live = sj[j] == kLive && __builtin_isfinite(lv[j]);
    const float p = live ? expf(lv[j] - mx) : 0.0f;
    ssum += p;
    hi[j] = bf16_rne_bits(p);
    lo[j] = bf16_rne_bits(p - bf16_bits_to_float(hi[j]));
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) ssum += __shfl_xor(ssum, o);
  const uint32_t w32 = a.chunks[r] * kAttnChunk;
  const uint64_t pidx = a.p_base[r] + static_cast<uint64_t>(head) * w32 + c * kAttnChunk + 4 * part;
  *reinterpret_cast<u16x4 *>(a.p_hi + pidx) = hi;
  *reinterpret_cast<u16x4 *>(a.p_lo + pidx) = lo;
  if (part == 0)
    a.stats[a.stat_base[r] + static_cast<uint64_t>(c) * kHeads + head] =
        make_float4(mx, ssum, bad ? 1.0f : 0.0f, sink_h);
}

// ---------------------------------------------------------------- phase 2
__global__ __launch_bounds__(kAttnThreads) void attn_reduce_kernel(AttnArgs a) {
  __shared__ float red[4 * kHeads * kRedStride];
  __shared__ __attribute__((aligned(16))) float fac[kChunksPerSuper * kHeads];
  __shared__ uint32_t s_bad[kHeads];

  // Row r on XCD r (block b = 8 dc + r): the row's probability planes,
  // statistics and G^T are read by all 16 feature chunks through one L2.
  const uint32_t r = blockIdx.x % kXcds;
  const uint32_t dc = blockIdx.x / kXcds;
  if (r >= a.rows) return;
  const uint32_t width = a.width[r];
  const uint32_t nch = a.chunks[r];
  const uint32_t w32 = nch * kAttnChunk;
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;
  const uint32_t hh = wave & 1;          // heads 32*hh ..
  const uint32_t sq = wave >> 1;         // chunks sq, sq+4, ... of each 512-slot span
  const uint32_t col = lane & 31;
  const uint32_t g = lane >> 5;
  const float4 *stats = a.stats + a.stat_base[r];
  const uint32_t head = tid >> 3, part = tid & 7;   // statistics work split

  const uint32_t ahead = 32 * hh + col;             // A row of this lane
  const uint16_t *phi = a.p_hi + a.p_base[r] + static_cast<uint64_t>(ahead) * w32;
  const uint16_t *plo = a.p_lo + a.p_base[r] + static_cast<uint64_t>(ahead) * w32;
  const uint16_t *gtr = a.gt + a.gt_base[r] + static_cast<uint64_t>(dc * kAttnDimChunk + col) * w32;

  f32x16 out = {};
  float m = 0.0f, invz = 0.0f;
  for (uint32_t s0 = 0; s0 < width; s0 += kAttnSuper) {
    const uint32_t c0 = s0 / kAttnChunk;
    const uint32_t span_chunks = min(nch - c0, static_cast<uint32_t>(kChunksPerSuper));
    // Statistics of the span's chunks first (8 threads per head, 2 chunks
    // each), then this wave's operands, all loads in flight together. Loads
    // complete in issue order, so waiting for the statistics leaves the
    // operand loads in flight.
    // (Unconditional loads from clamped, always valid, chunk indices.)
    const float4 x0 = stats[static_cast<uint64_t>(min(c0 + part, nch - 1)) * kHeads + head];
    const float4 x1 = stats[static_cast<uint64_t>(min(c0 + part + 8, nch - 1)) * kHeads + head];
    u32x4 ah[4][2], al[4][2], bv[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t cc = sq + 4 * j;
      const uint32_t ccl = min(cc, span_chunks - 1);   // unconditional loads; unused past the span
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t sl = s0 + ccl * kAttnChunk + 16 * k + 8 * g;
        ah[j][k] = load16(phi + sl);
        al[j][k] = load16(plo + sl);
        bv[j][k] = load16(gtr + sl);
      }
    }
    const float4 none = make_float4(-__builtin_inff(), 0.0f, 0.0f, 0.0f);
    const float4 st0 = part < span_chunks ? x0 : none;
    const float4 st1 = part + 8 < span_chunks ? x1 : none;
    if (s0 == 0) {
      // m, Z and the bad flag of each head need every chunk: those of the
      // first span are in registers; rows wider than one span read the rest.
      const float sink = x0.w;   // phase 1 stores each head's sink with its statistics
      bool bad = !__builtin_isfinite(sink);
      float mm = bad ? 0.0f : sink;
      auto take_max = [&](const float4 &x) {
        bad |= x.z != 0.0f;
        if (x.y > 0.0f) mm = fmaxf(mm, x.x);
      };
      take_max(st0);
      take_max(st1);
      for (uint32_t cc = kChunksPerSuper + part; cc < nch; cc += 8) take_max(stats[static_cast<uint64_t>(cc) * kHeads + head]);
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        mm = fmaxf(mm, __shfl_xor(mm, o));
        const int other = __shfl_xor(static_cast<int>(bad), o);   // every lane must take part
        bad = bad || other != 0;
      }
      float z = 0.0f;
      auto take_sum = [&](const float4 &x) {
        if (x.y > 0.0f) z += x.y * expf(x.x - mm);
      };
      take_sum(st0);
      take_sum(st1);
      for (uint32_t cc = kChunksPerSuper + part; cc < nch; cc += 8) take_sum(stats[static_cast<uint64_t>(cc) * kHeads + head]);
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) z += __shfl_xor(z, o);
      z += bad ? 0.0f : expf(sink - mm);
      bad |= !(z > 0.0f && __builtin_isfinite(z));
      m = mm;
      invz = bad ? 0.0f : 1.0f / z;
      if (part == 0) s_bad[head] = bad ? 1u : 0u;
    }
    __syncthreads();   // previous span's factor reads are done
    fac[part * kHeads + head] = st0.y > 0.0f ? expf(st0.x - m) * invz : 0.0f;
    fac[(part + 8) * kHeads + head] = st1.y > 0.0f ? expf(st1.x - m) * invz : 0.0f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t cc = sq + 4 * j;
      if (cc < span_chunks) {
        f32x16 acc = {};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          acc = mfma32(as_bf16x8(ah[j][k]), as_bf16x8(bv[j][k]), acc);
          acc = mfma32(as_bf16x8(al[j][k]), as_bf16x8(bv[j][k]), acc);
        }
        const f32x4 *fr = reinterpret_cast<const f32x4 *>(&fac[cc * kHeads + 32 * hh + 4 * g]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 f = fr[2 * q];      // heads 32hh + 8q + 4g .. +4
#pragma unroll
          for (int i = 0; i < 4; ++i) out[4 * q + i] = fmaf(f[i], acc[4 * q + i], out[4 * q + i]);
        }
      }
    }
  }

  // Sum the four chunk-set partials in a fixed order.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t h = 32 * hh + 8 * (i / 4) + 4 * g + (i % 4);
    red[(sq * kHeads + h) * kRedStride + col] = out[i];
  }
  __syncthreads();
  const uint64_t obase = static_cast<uint64_t>(a.q_row[r]) * kHeads * kDim + dc * kAttnDimChunk;
  for (uint32_t i = tid; i < kHeads * kAttnDimChunk; i += kAttnThreads) {
    const uint32_t h = i / kAttnDimChunk, d = i % kAttnDimChunk;
    float v = red[(0 * kHeads + h) * kRedStride + d];
    v += red[(1 * kHeads + h) * kRedStride + d];
    v += red[(2 * kHeads + h) * kRedStride + d];
    v += red[(3 * kHeads + h) * kRedStride + d];
    a.out[obase + static_cast<uint64_t>(h) * kDim + d] = (s_bad[h] == 0 && __builtin_isfinite(v)) ? v : 0.0f;
  }
}

hipError_t launch_attn_logits(const AttnArgs &a, bool direct, uint32_t blocks, hipStream_t s) {
  if (direct)
    hipLaunchKernelGGL(attn_logits_kernel<true>, dim3(blocks), dim3(kAttnThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_logits_kernel<false>, dim3(blocks), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_reduce(const AttnArgs &a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(attn_reduce_kernel, dim3(blocks), dim3(kAttnThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
