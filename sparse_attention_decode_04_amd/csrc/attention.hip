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
// Two launches (split over the selected slots, then a combine). The selected
// rows G[t] come either from the gathered operand and its mask (after
// ds_rows_gather) or, in the direct variant, straight from each row's KV
// through the indices (the gather fused in).
//   phase 1, per (row, 64-slot chunk c), 8 waves: the query (64 KiB) and
//     the chunk's rows (64 KiB) are loaded once each, into LDS; the logits
//     on MFMA 32x32x16 (M = 32 heads, N = 32 slots, K = 16 features), four
//     waves each taking one 32x32 tile over all 512 features. Per head: the
//     chunk max m_c, p~ = exp(l - m_c) as a bf16 pair
//     (hi = bf16(p~), lo = bf16(p~ - hi): ~16 significant bits) and
//     s_c = sum p~. Then the chunk's output O_c = p~ . G_c (64 heads x 512
//     features, f32) on MFMA 16x16x32 (M = 16 heads, N = 16 features,
//     K = 32 slots), each wave owning 64 features. The chunk's rows stay in
//     LDS as loaded (slot-major); the B operand, 8 consecutive slots of one
//     feature per lane, comes from two transposing LDS reads
//     (ds_read_b64_tr_b16: within each 16-lane group, lane i receives the
//     i-th 16-bit element of the 8-byte pieces that lanes 4k + i/4 address,
//     k = 0..3).
//   phase 2, per (row, 32-feature chunk), 4 waves: m, Z and the bad flag of
//     each head from the chunk statistics and the sink, then
//     out = sum_c e^(m_c - m) O_c / Z in a fixed chunk order.
// All splits depend only on the row's own width, so rows are independent
// bit for bit, and both variants give the same bits.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

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
// Transposing 8-byte LDS read (see the header comment for its lane layout).
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
}

constexpr int kChunkThreads = 512;              // 8 waves
constexpr int kRowStride = kDim + 8;            // bf16 per LDS row of q and of the chunk's rows: 1040 B
constexpr int kRedStride = kAttnChunk + 1;      // padded f32 row of the logits
constexpr int kPStride = kAttnChunk + 8;        // bf16 per LDS head row of p~: 144 B
constexpr int kCombineThreads = 256;
// LDS of phase 1: the chunk's rows, and one region that holds the query
// during the logits and then the logits and p~.
constexpr int kVtBytes = kAttnChunk * kRowStride * 2;                  // 66,560
constexpr int kQBytes = kHeads * kRowStride * 2;                       // 66,560
constexpr int kRedBytes = kHeads * kRedStride * 4;                     // 16,640
constexpr int kPBytes = kHeads * kPStride * 2;                         // 9,216
static_assert(kRedBytes + 2 * kPBytes <= kQBytes, "logits and p~ fit over the query");

// ---------------------------------------------------------------- phase 1
template <bool kDirect>
__global__ __launch_bounds__(kChunkThreads) void attn_chunk_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kVtBytes / 2];   // the chunk's rows, slot-major
  __shared__ __attribute__((aligned(16))) unsigned char ureg[kQBytes];
  __shared__ uint32_t state[kAttnChunk];
  uint16_t *q_lds = reinterpret_cast<uint16_t *>(ureg);                  // query [64][kRowStride]
  float *red = reinterpret_cast<float *>(ureg);                          // logits [64][kRedStride]
  uint16_t *phi = reinterpret_cast<uint16_t *>(ureg + kRedBytes);        // p~ hi [64][kPStride]
  uint16_t *plo = reinterpret_cast<uint16_t *>(ureg + kRedBytes + kPBytes);

  // Row r runs on XCD r (consecutive workgroups go to consecutive XCDs), so
  // all chunks of a row share one L2.
  const uint32_t r = blockIdx.x % kXcds;
  const uint32_t c = blockIdx.x / kXcds;
  if (r >= a.rows || c >= a.chunks[r]) return;
  const uint32_t width = a.width[r];
  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tid >> 6;

  // Loads: thread t moves features 64 (t % 8) .. +64 of slot t / 8 and of
  // head t / 8 of the query, each byte once. They are unconditional (a slot
  // past the width reads the row's last slot, a sentinel or bad index reads
  // KV row 0) and masked afterwards, so they are all in flight at once. The
  // slot's index (or mask entry) goes first: the KV row load depends on it,
  // and loads complete in issue order.
  const uint32_t sl = tid >> 3;            // slot within the chunk (and query head)
  const uint32_t fp = 64 * (tid & 7);      // this thread's 64 features
  const uint32_t slot = c * kAttnChunk + sl;
  const uint32_t cslot = min(slot, width - 1);
  int32_t raw_index = 0;
  uint16_t raw_mask = 0;
  if (kDirect) raw_index = a.indices[a.index_offset[r] + cslot];
  else raw_mask = a.mask[a.slot_base[r] + cslot];
  const uint16_t *qrow = a.q + (static_cast<uint64_t>(a.q_row[r]) * kHeads + sl) * kDim + fp;
  u32x4 qv[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qv[s] = load16(qrow + 8 * s);
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
  // The sink of head t / 8 (the epilogue's head), stored with the chunk
  // statistics so that phase 2 gets it in the same load.
  const float sink_h = a.sinks[tid >> 3];
  u32x4 gb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) gb[s] = load16(src + fp + 8 * s);
#pragma unroll
  for (int s = 0; s < 8; ++s)
    if (!use) gb[s] = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    *reinterpret_cast<u32x4 *>(&q_lds[sl * kRowStride + fp + 8 * s]) = qv[s];
    *reinterpret_cast<u32x4 *>(&vt[sl * kRowStride + fp + 8 * s]) = gb[s];
  }
  if (kDirect) {
    // Gather semantics: a non-finite element makes the row invalid. The eight
    // threads of a slot are eight consecutive lanes.
    bool nf = false;
#pragma unroll
    for (int s = 0; s < 8; ++s) nf |= any_nonfinite(gb[s]);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const int other = __shfl_xor(static_cast<int>(nf), o);   // every lane must take part
      nf = nf || other != 0;
    }
    if (st == kLive && nf) st = kBad;
  }
  if ((tid & 7) == 0) state[sl] = st;
  __syncthreads();

  // Logits on MFMA 32x32x16, full K = 512 per tile: waves 0..3 take the tiles
  // (heads 32 (w % 2) .., slots 32 (w / 2) ..); operands from LDS, lane l
  // reading row l % 32 at features 16 j + 8 (l / 32) in step j.
  f32x16 acc = {};
  const uint32_t col = lane & 31;
  const uint32_t g = lane >> 5;
  const uint32_t th = 32 * (wave & 1), ts = 32 * ((wave >> 1) & 1);
  if (wave < 4) {
    const uint16_t *qa = &q_lds[(th + col) * kRowStride + 8 * g];
    const uint16_t *kb = &vt[(ts + col) * kRowStride + 8 * g];
#pragma unroll
    for (int j = 0; j < kDim / 16; ++j)
      acc = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(qa + 16 * j)),
                   as_bf16x8(*reinterpret_cast<const u32x4 *>(kb + 16 * j)), acc);
  }
  __syncthreads();   // the query region becomes the logits
  if (wave < 4) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      red[(th + 8 * (i / 4) + 4 * g + (i % 4)) * kRedStride + ts + col] = acc[i];
  }
  __syncthreads();

  // Softmax statistics. Thread t: head t / 8, slots 8 * (t % 8) .. +8.
  {
    const uint32_t head = tid >> 3;
    const uint32_t part = tid & 7;
    float lv[8];
    uint32_t sj[8];
    bool bad = false;
    float mx = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t s = 8 * part + j;
      lv[j] = red[head * kRedStride + s] * a.scale;
      sj[j] = state[s];
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
    u16x8 hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool live = sj[j] == kLive && __builtin_isfinite(lv[j]);
      const float p = live ? expf(lv[j] - mx) : 0.0f;
      ssum += p;
      hi[j] = bf16_rne_bits(p);
      lo[j] = bf16_rne_bits(p - bf16_bits_to_float(hi[j]));
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) ssum += __shfl_xor(ssum, o);
    *reinterpret_cast<u16x8 *>(&phi[head * kPStride + 8 * part]) = hi;
    *reinterpret_cast<u16x8 *>(&plo[head * kPStride + 8 * part]) = lo;
    if (part == 0)
      a.stats[a.stat_base[r] + static_cast<uint64_t>(c) * kHeads + head] =
          make_float4(mx, ssum, bad ? 1.0f : 0.0f, sink_h);
  }
  __syncthreads();

  // O_c = p~ . G_c: this wave's 64 features, all 64 heads, K = 64 slots.
  const uint32_t li = lane & 15;
  const uint32_t lg = lane >> 4;
  f32x4 o[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) o[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8 ahi[4], alo[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint32_t off = (16 * mt + li) * kPStride + 32 * ks + 8 * lg;   // head 16mt + li, slots ..+8
      ahi[mt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&phi[off]));
      alo[mt] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&plo[off]));
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      // Lane li of group lg receives features n0 + li of slots s0 .. s0+3
      // and s0+4 .. s0+7 (s0 = 32 ks + 8 lg): it addresses slot s0 + li/4
      // (+4), features n0 + 4 (li % 4) .. +4.
      const uint32_t n0 = 64 * wave + 16 * nt;
      const uint32_t s0 = 32 * ks + 8 * lg;
      const s16x4 b0 = lds_read_tr16(&vt[(s0 + li / 4) * kRowStride + n0 + 4 * (li % 4)]);
      const s16x4 b1 = lds_read_tr16(&vt[(s0 + 4 + li / 4) * kRowStride + n0 + 4 * (li % 4)]);
      const s16x8 b8 = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      const bf16x8 b = __builtin_bit_cast(bf16x8, b8);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        o[mt][nt] = mfma16(ahi[mt], b, o[mt][nt]);
        o[mt][nt] = mfma16(alo[mt], b, o[mt][nt]);
      }
    }
  }
  // D lane l of tile (mt, nt): feature 64 wave + 16 nt + l % 16, heads
  // 16 mt + 4 (l / 16) + i.
  float *dst = a.opart + a.part_base[r] + static_cast<uint64_t>(c) * kHeads * kDim;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[(16 * mt + 4 * lg + i) * kDim + 64 * wave + 16 * nt + li] = o[mt][nt][i];
}

// ---------------------------------------------------------------- phase 2
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(AttnArgs a) {
  // Row r on XCD r (block b = 8 dc + r), as in phase 1.
  const uint32_t r = blockIdx.x % kXcds;
  const uint32_t dc = blockIdx.x / kXcds;
  if (r >= a.rows) return;
  const uint32_t nch = a.chunks[r];
  const uint32_t tid = threadIdx.x;
  const uint32_t head = tid >> 2;
  const uint32_t d0 = kAttnDimChunk * dc + 8 * (tid & 3);
  const float4 *stats = a.stats + a.stat_base[r] + head;
  const float *op = a.opart + a.part_base[r] + static_cast<uint64_t>(head) * kDim + d0;
  constexpr int kB = 8;   // chunks per batch of loads
  auto stat_at = [&](uint32_t cc) { return stats[static_cast<uint64_t>(min(cc, nch - 1)) * kHeads]; };
  auto part_at = [&](uint32_t cc, int half) {
    return *reinterpret_cast<const f32x4 *>(op + static_cast<uint64_t>(min(cc, nch - 1)) * kHeads * kDim + 4 * half);
  };

  // First batch of statistics and outputs, all loads in flight at once.
  float4 x[kB];
  f32x4 p0[kB], p1[kB];
#pragma unroll
  for (int i = 0; i < kB; ++i) x[i] = stat_at(i);
#pragma unroll
  for (int i = 0; i < kB; ++i) { p0[i] = part_at(i, 0); p1[i] = part_at(i, 1); }

  // m, the bad flag and Z over all chunks, with the sink.
  const float sink = x[0].w;   // phase 1 stores the head's sink with every statistic
  bool bad = !__builtin_isfinite(sink);
  float m = bad ? 0.0f : sink;
  auto take_max = [&](const float4 &s) {
    bad |= s.z != 0.0f;
    if (s.y > 0.0f) m = fmaxf(m, s.x);
  };
#pragma unroll
  for (int i = 0; i < kB; ++i)
    if (static_cast<uint32_t>(i) < nch) take_max(x[i]);
  for (uint32_t cc = kB; cc < nch; ++cc) take_max(stat_at(cc));
  float z = bad ? 0.0f : expf(sink - m);
  auto weight = [&](const float4 &s) { return s.y > 0.0f ? expf(s.x - m) : 0.0f; };
#pragma unroll
  for (int i = 0; i < kB; ++i)
    if (static_cast<uint32_t>(i) < nch) z += x[i].y * weight(x[i]);
  for (uint32_t cc = kB; cc < nch; ++cc) {
    const float4 s = stat_at(cc);
    z += s.y * weight(s);
  }
  bad |= !(z > 0.0f && __builtin_isfinite(z));

  f32x4 acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kB; ++i) {
    const float w = static_cast<uint32_t>(i) < nch ? weight(x[i]) : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc0[k] = fmaf(w, p0[i][k], acc0[k]);
      acc1[k] = fmaf(w, p1[i][k], acc1[k]);
    }
  }
  for (uint32_t cc = kB; cc < nch; ++cc) {
    const float w = weight(stat_at(cc));
    const f32x4 q0 = part_at(cc, 0), q1 = part_at(cc, 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc0[k] = fmaf(w, q0[k], acc0[k]);
      acc1[k] = fmaf(w, q1[k], acc1[k]);
    }
  }
  const float invz = bad ? 0.0f : 1.0f / z;
  f32x4 v0, v1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float u0 = acc0[k] * invz, u1 = acc1[k] * invz;
    v0[k] = (!bad && __builtin_isfinite(u0)) ? u0 : 0.0f;
    v1[k] = (!bad && __builtin_isfinite(u1)) ? u1 : 0.0f;
  }
  float *dst = a.out + (static_cast<uint64_t>(a.q_row[r]) * kHeads + head) * kDim + d0;
  *reinterpret_cast<f32x4 *>(dst) = v0;
  *reinterpret_cast<f32x4 *>(dst + 4) = v1;
}

hipError_t launch_attn_chunks(const AttnArgs &a, bool direct, uint32_t blocks, hipStream_t s) {
  if (direct)
    hipLaunchKernelGGL(attn_chunk_kernel<true>, dim3(blocks), dim3(kChunkThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_chunk_kernel<false>, dim3(blocks), dim3(kChunkThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnArgs &a, uint32_t blocks, hipStream_t s) {
  hipLaunchKernelGGL(attn_combine_kernel, dim3(blocks), dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ds
