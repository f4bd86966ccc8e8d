// Phase 1 of the sparse attention for one (row, head group, 64-slot chunk):
// shared state, helpers and the body, used by the attention kernel and by the
// kernel that runs a row's final top-k level ahead of it. (The method is
// described at the top of attention.hip.)
#pragma once

#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Slot states: -inf mask / -1 index = sentinel (dropped), bad index or a
// non-finite KV element (direct variant) = bad (the row is zeroed).
enum : uint32_t { kLive = 0, kSkip = 1, kBad = 2 };

// Workgroup (x, r) of the phase-1 grid: chunk c and head group hg of row r.
__device__ __forceinline__ void attn_block(uint32_t x, uint32_t &c, uint32_t &hg) {
  hg = (x / kXcds) % kAttnHeadGroups;
  c = kXcds * (x / (kXcds * kAttnHeadGroups)) + x % kXcds;
}

__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Whether any of the eight bf16 in v is not finite (exponent bits all ones).
// Per 32-bit word: the exponent fields of both halves plus 0x80 each carry
// into bit 15 of their half exactly when they are all ones (no carry crosses
// into the upper half), so one mask, one add and one test cover two values.
__device__ __forceinline__ bool any_nonfinite(u32x4 v) {
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) c |= (v[k] & 0x7F807F80u) + 0x00800080u;
  return (c & 0x80008000u) != 0;
}
// Transposing 8-byte LDS read (see the header comment for its lane layout).
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
}

constexpr int kChunkThreads = 1024;             // 16 waves
constexpr int kHg = kHeads / kAttnHeadGroups;   // heads per phase-1 workgroup (16)
constexpr int kRowStride = kDim + 8;            // bf16 per LDS row of q and of the chunk's rows: 1040 B
constexpr int kRedStride = kAttnChunk + 1;      // padded f32 row of the logits
constexpr int kPStride = kAttnChunk + 8;        // bf16 per LDS head row of p~: 144 B
static_assert(kHg == 16, "one MFMA row tile of heads per workgroup");

// ---------------------------------------------------------------- phase 1
// The chunk's LDS: its rows, the group's query heads, the logits, p~.
struct AttnChunkShared {
  __attribute__((aligned(16))) uint16_t vt[kAttnChunk * kRowStride];   // the chunk's rows, slot-major
  __attribute__((aligned(16))) uint16_t q_lds[kHg * kRowStride];       // this group's query heads
  float red[(kChunkThreads / 256) * kHg * kRedStride];                  // logits, one plane per K part
  __attribute__((aligned(16))) uint16_t phi[kHg * kPStride];            // p~ hi
  __attribute__((aligned(16))) uint16_t plo[kHg * kPStride];            // p~ lo
  uint32_t state[kAttnChunk];
  float madd[kAttnChunk];   // gathered variant: the mask value added to a live slot's logit
};

// One row's arguments of phase 1, read in one batch (see LevelRow: each
// read on its own would cost a dependent scalar-load round trip).
struct AttnRow {
  const uint16_t *rows;     // direct: the row's KV; gathered: its gathered rows
  const uint16_t *mask;     // gathered: the row's mask entries
  const uint32_t *invalid;  // gathered: the row's invalid flag
  const uint16_t *q;        // the row's query [64, 512]
  const float *sinks;
  float4 *stats;            // the row's chunk statistics
  float *opart;             // the row's chunk outputs
  uint32_t width;
  uint32_t kv_len;
  float scale;
};

// Row r's AttnRow; x0, x1 (32-bit), x2 (64-bit) and x3 (32-bit) are more
// arguments of the caller read in the same batch (in as values read from the
// arguments, out unchanged).
template <bool kDirect>
__device__ __forceinline__ AttnRow attn_row(const AttnArgs &a, uint32_t r, uint32_t &x0, uint32_t &x1, uint64_t &x2,
                                            uint32_t &x3) {
  uint64_t rows = reinterpret_cast<uint64_t>(kDirect ? a.kv[r] : a.gathered);
  uint64_t mask = reinterpret_cast<uint64_t>(a.mask), slot_base = kDirect ? 0 : a.slot_base[r];
  uint64_t inv = reinterpret_cast<uint64_t>(a.invalid);
  uint64_t q = reinterpret_cast<uint64_t>(a.q), sinks = reinterpret_cast<uint64_t>(a.sinks);
  uint64_t stats = reinterpret_cast<uint64_t>(a.stats), stat_base = a.stat_base[r];
  uint64_t opart = reinterpret_cast<uint64_t>(a.opart), part_base = a.part_base[r];
  uint32_t q_row = a.q_row[r], width = a.width[r], kv_len = a.kv_len[r], scale = __float_as_uint(a.scale);
  asm volatile("" : "+s"(rows), "+s"(mask), "+s"(slot_base), "+s"(inv), "+s"(q), "+s"(sinks), "+s"(stats), "+s"(stat_base),
               "+s"(opart), "+s"(part_base), "+s"(q_row), "+s"(width), "+s"(kv_len), "+s"(scale), "+s"(x0), "+s"(x1),
               "+s"(x2), "+s"(x3));
  AttnRow ar;
  ar.rows = global_ptr<const uint16_t>(rows) + slot_base * kDim;
  ar.mask = global_ptr<const uint16_t>(mask) + slot_base;
  ar.invalid = global_ptr<const uint32_t>(inv) + r;
  ar.q = global_ptr<const uint16_t>(q) + static_cast<uint64_t>(q_row) * kHeads * kDim;
  ar.sinks = global_ptr<const float>(sinks);
  ar.stats = global_ptr<float4>(stats) + stat_base;
  ar.opart = global_ptr<float>(opart) + part_base;
  ar.width = width;
  ar.kv_len = kv_len;
  ar.scale = __uint_as_float(scale);
  return ar;
}

// The softmax normaliser of one head over its row's chunks, from each
// chunk's statistics s_c = (m_c, sum_c, bad_c, sink) in chunk order:
// m = max(sink, m_c of chunks with a live slot), Z = exp(sink - m) +
// sum_c sum_c exp(m_c - m); the head is bad when the sink, a chunk or Z is.
// Every multiply-add is an explicit fmaf (the combine's bits do not depend
// on how the compiler contracts the code around it).
struct HeadNorm {
  float m, invz;   // invz = 1/Z, or 0 for a bad head
  bool bad;
};
__device__ __forceinline__ float chunk_weight(const float4 &s, float m) { return s.y > 0.0f ? expf(s.x - m) : 0.0f; }
// first_at(cc) gives the statistics of the first kUnrolled chunks (called
// with compile-time cc, so statistics held in register arrays stay in
// registers), later_at(cc) those of the rest; chunks are taken in order.
// w_first[cc] receives the weight of each of the first kUnrolled chunks (0
// past the row's chunks), so that the weighted sum need not recompute them.
// The unrolled part selects rather than branches on cc < nch.
template <int kUnrolled, class FirstAt, class LaterAt>
__device__ __forceinline__ HeadNorm head_norm(float sink, uint32_t nch, const FirstAt &first_at,
                                              const LaterAt &later_at, float (&w_first)[kUnrolled]) {
  bool bad = !__builtin_isfinite(sink);
  float m = bad ? 0.0f : sink;
  auto take_max = [&](const float4 &s) {
    bad |= s.z != 0.0f;
    if (s.y > 0.0f) m = fmaxf(m, s.x);
  };
#pragma unroll
  for (int cc = 0; cc < kUnrolled; ++cc) {
    const float4 s = first_at(cc);
    const bool in = static_cast<uint32_t>(cc) < nch;
    bad |= in && s.z != 0.0f;
    m = (in && s.y > 0.0f) ? fmaxf(m, s.x) : m;
  }
  for (uint32_t cc = kUnrolled; cc < nch; ++cc) take_max(later_at(cc));
  float z = bad ? 0.0f : expf(sink - m);
#pragma unroll
  for (int cc = 0; cc < kUnrolled; ++cc) {
    const float4 s = first_at(cc);
    const bool in = static_cast<uint32_t>(cc) < nch;
    w_first[cc] = in ? chunk_weight(s, m) : 0.0f;
    z = in ? fmaf(s.y, w_first[cc], z) : z;
  }
  for (uint32_t cc = kUnrolled; cc < nch; ++cc) {
    const float4 s = later_at(cc);
    z = fmaf(s.y, chunk_weight(s, m), z);
  }
  bad |= !(z > 0.0f && __builtin_isfinite(z));
  return HeadNorm{m, bad ? 0.0f : 1.0f / z, bad};
}
// One output element from its weighted sum: acc / Z, zeroed for a bad head
// or a non-finite value.
__device__ __forceinline__ float head_out(float acc, float invz, bool bad) {
  const float u = acc * invz;
  return (!bad && __builtin_isfinite(u)) ? u : 0.0f;
}

// Phase 1 for (row r, head group hg, chunk c) by the first kChunkThreads
// threads of the workgroup (further waves of a wider workgroup would only
// take part in the barriers). raw_index_at(slot) gives the direct variant the
// index of one of the row's slots (slot < width).
template <bool kDirect, class RawIndex>
__device__ __forceinline__ void attn_chunk_body(AttnChunkShared &sm, const AttnRow &a, uint32_t hg, uint32_t c,
                                                const RawIndex &raw_index_at) {
  uint16_t *const vt = sm.vt;
  uint16_t *const q_lds = sm.q_lds;
  float *const red = sm.red;
  uint16_t *const phi = sm.phi;
  uint16_t *const plo = sm.plo;
  uint32_t *const state = sm.state;
  const uint32_t width = a.width;
  const uint32_t tid = threadIdx.x;
  const bool active = tid < static_cast<uint32_t>(kChunkThreads);   // wave-uniform
  const uint32_t lane = tid & 63;
  // Wave-uniform (as a scalar, so that slot and row arithmetic stays scalar).
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int kTph = kChunkThreads / kHg;   // softmax threads per head: 32 or 64
  const uint32_t qh = tid / kTph;              // the softmax head of this thread
  // The sink of the softmax head, stored with the chunk statistics so that
  // phase 2 gets it in the same load.
  const float sink_h = active ? a.sinks[kHg * hg + qh] : 0.0f;
  // Gathered variant: the row's invalid flag, read by every thread with its
  // other first loads and used in the softmax.
  const bool row_invalid = !kDirect && active && *a.invalid != 0;
  constexpr int kSlots = kAttnChunk / (kChunkThreads / 64);   // slots per wave: 8 or 4
  constexpr int kQHeads = kHg / (kChunkThreads / 64);         // query heads per wave: 2 or 1
  static_assert(kChunkThreads == 512 || kChunkThreads == 1024, "8 or 16 waves");

  if (active) {
    // Loads: wave w moves kSlots slots (kSlots w ..) of the chunk and kQHeads
    // query heads of the group, one whole 1 KiB row per load instruction
    // (lane l: features 8l .. 8l + 8), each byte once. They are
    // unconditional (a slot past the width reads the row's last slot, a
    // sentinel or bad index reads KV row 0) and masked afterwards, so they
    // are all in flight at once. The slots' indices (or mask entries) come
    // first: the row loads depend on them.
    const uint32_t s0 = c * kAttnChunk + kSlots * wave;   // first slot of this wave
    int32_t raw_index[kSlots];
    uint16_t raw_mask[kSlots];
  #pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const uint32_t cslot = min(s0 + s, width - 1);
      // Every lane reads the same slot. The direct variant keeps the index
      // in a vector register (an opaque per-lane copy), so that the checks
      // and the 64-bit row address below run on the vector ALUs, each SIMD
      // for its own waves: as wave-uniform scalar code they would queue
      // every wave of the workgroup on the compute unit's one scalar ALU.
      if (kDirect) raw_index[s] = raw_index_at(cslot);
      else raw_mask[s] = a.mask[cslot];
    }
    if (kDirect) {
  #pragma unroll
      for (int s = 0; s < kSlots; ++s) asm volatile("" : "+v"(raw_index[s]));
    }
    // The row's fields once, out of the loop below. An index i is live when
    // 0 <= i < kv_len, i.e. when it is below min(kv_len, 2^31) as an
    // unsigned number (one compare); past the width it reads as -1 (skip).
    const uint32_t kv_lim = min(a.kv_len, 0x80000000u);
    const uint16_t *const lane_row0 = a.rows + 8 * lane;   // this lane's 16 bytes of KV row 0
    uint32_t st[kSlots];
    bool use[kSlots];
    const uint16_t *src[kSlots];
  #pragma unroll
    for (int s = 0; s < kSlots; ++s) {
      const uint32_t slot = s0 + s;
      if (kDirect) {
        const int32_t i = slot < width ? raw_index[s] : -1;
        const uint32_t iu = static_cast<uint32_t>(i);
        const bool ok = iu < kv_lim;
        st[s] = ok ? kLive : (i != -1 ? kBad : kSkip);
        src[s] = lane_row0 + static_cast<uint64_t>(ok ? iu : 0u) * kDim;
      } else {
        st[s] = (slot < width && raw_mask[s] != kBf16NegInf) ? kLive : kSkip;
        src[s] = lane_row0 + static_cast<uint64_t>(min(slot, width - 1)) * kDim;
      }
      use[s] = kDirect ? st[s] == kLive : slot < width;
    }
    u32x4 gb[kSlots];
  #pragma unroll
    for (int s = 0; s < kSlots; ++s) gb[s] = load16(src[s]);
    const uint16_t *qbase = a.q + (kHg * hg + kQHeads * wave) * kDim + 8 * lane;
    u32x4 qv[kQHeads];
  #pragma unroll
    for (int h = 0; h < kQHeads; ++h) qv[h] = load16(qbase + h * kDim);
    // Every load is issued before any of their results is used (the
    // scheduler would otherwise pull the masking of the first rows up
    // between the loads, with a wait for them that holds back the rest).
    __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
    for (int s = 0; s < kSlots; ++s)
      if (!use[s]) gb[s] = u32x4{0, 0, 0, 0};
  #pragma unroll
    for (int h = 0; h < kQHeads; ++h) *reinterpret_cast<u32x4 *>(&q_lds[(kQHeads * wave + h) * kRowStride + 8 * lane]) = qv[h];
  #pragma unroll
    for (int s = 0; s < kSlots; ++s) *reinterpret_cast<u32x4 *>(&vt[(kSlots * wave + s) * kRowStride + 8 * lane]) = gb[s];
    if (kDirect) {
      // Gather semantics: a non-finite element makes the row invalid.
  #pragma unroll
      for (int s = 0; s < kSlots; ++s)
        if (st[s] == kLive && __ballot(any_nonfinite(gb[s])) != 0) st[s] = kBad;
    }
    if (lane == 0) {
  #pragma unroll
      for (int s = 0; s < kSlots; ++s) state[kSlots * wave + s] = st[s];
      if (!kDirect) {
  #pragma unroll
        for (int s = 0; s < kSlots; ++s) sm.madd[kSlots * wave + s] = bf16_bits_to_float(raw_mask[s]);
      }
    }
  }
  __syncthreads();

  if (active) {
    // Logits on MFMA 16x16x32 (M = 16 heads, N = 16 slots, K = 32 features):
    // wave w takes slots 16 (w % 4) .. +16 and K part w / 4 of kKParts
    // (kKLen features, kKLen / 32 steps); lane l reads row l % 16 at features
    // 32 j + 8 (l / 16) of step j. Each part goes to its own plane; the
    // softmax adds the planes in part order.
    {
      constexpr int kKParts = kChunkThreads / 256;   // 2 or 4
      constexpr int kKLen = kDim / kKParts;
      const uint32_t col = lane & 15;
      const uint32_t grp = lane >> 4;
      const uint32_t ts = 16 * (wave & 3), kh = wave >> 2;
      const uint16_t *qa = &q_lds[col * kRowStride + kKLen * kh + 8 * grp];
      const uint16_t *kb = &vt[(ts + col) * kRowStride + kKLen * kh + 8 * grp];
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  #pragma unroll
      for (int j = 0; j < kKLen / 32; ++j)
        acc = mfma16(as_bf16x8(*reinterpret_cast<const u32x4 *>(qa + 32 * j)),
                     as_bf16x8(*reinterpret_cast<const u32x4 *>(kb + 32 * j)), acc);
      // D lane l: slot ts + l % 16, heads 4 (l / 16) + i.
  #pragma unroll
      for (int i = 0; i < 4; ++i) red[(kh * kHg + 4 * grp + i) * kRedStride + ts + col] = acc[i];
    }
  }
  __syncthreads();

  if (active) {
    // Softmax statistics. Thread t: head t / kTph, slots kSpt (t % kTph) ..
    // + kSpt (with 16 waves: one wave per head, one slot per thread).
    {
      // No contraction here: each logit is rounded once as scale * sum (plus
      // the mask entry in the gathered variant) before it is compared and
      // exponentiated, so that both variants give the same bits (a fused
      // multiply-subtract into the exponent would round differently).
#pragma clang fp contract(off)
      constexpr int kKParts = kChunkThreads / 256;
      constexpr int kSpt = kAttnChunk / kTph;   // slots per thread: 2 or 1
      const uint32_t head = qh;
      const uint32_t part = tid % kTph;
      float lv[kSpt];
      uint32_t sj[kSpt];
      bool bad = row_invalid;
      float mx = -__builtin_inff();
  #pragma unroll
      for (int j = 0; j < kSpt; ++j) {
        const uint32_t s = kSpt * part + j;
        float l = red[head * kRedStride + s];
  #pragma unroll
        for (int k = 1; k < kKParts; ++k) l += red[(k * kHg + head) * kRedStride + s];
        lv[j] = l * a.scale;
        if (!kDirect) lv[j] += sm.madd[s];   // additive mask: 0 for every slot ds_rows_gather keeps
        sj[j] = state[s];
        const bool live = sj[j] == kLive;
        bad |= (sj[j] == kBad) || (live && !__builtin_isfinite(lv[j]));
        if (live && __builtin_isfinite(lv[j])) mx = fmaxf(mx, lv[j]);
      }
      if constexpr (kTph == 32) {
        mx = half_max(mx);
        bad = half_any(bad);
      } else {
        mx = wave_max_f(mx);
        bad = __ballot(bad) != 0;
      }
      float ssum = 0.0f;
      uint32_t hi2 = 0, lo2 = 0;
  #pragma unroll
      for (int j = 0; j < kSpt; ++j) {
        const bool live = sj[j] == kLive && __builtin_isfinite(lv[j]);
        const float p = live ? expf(lv[j] - mx) : 0.0f;
        ssum += p;
        const uint16_t h = bf16_rne_bits(p);
        const uint16_t l = bf16_rne_bits(p - bf16_bits_to_float(h));
        hi2 |= static_cast<uint32_t>(h) << (16 * j);
        lo2 |= static_cast<uint32_t>(l) << (16 * j);
      }
      if constexpr (kTph == 32) {
        ssum = half_sum(ssum);
        *reinterpret_cast<uint32_t *>(&phi[head * kPStride + 2 * part]) = hi2;
        *reinterpret_cast<uint32_t *>(&plo[head * kPStride + 2 * part]) = lo2;
      } else {
        ssum = wave_sum_f(ssum);
        phi[head * kPStride + part] = static_cast<uint16_t>(hi2);
        plo[head * kPStride + part] = static_cast<uint16_t>(lo2);
      }
      if (part == 0)
        a.stats[static_cast<uint64_t>(c) * kHeads + kHg * hg + head] =
            make_float4(mx, ssum, bad ? 1.0f : 0.0f, sink_h);
    }
  }
  __syncthreads();

  if (active) {
    // O_c = p~ . G_c for the group's 16 heads: wave w's kFpw features, K = 64
    // slots (MFMA 16x16x32: M = 16 heads, N = 16 features, K = 32 slots).
    constexpr int kFpw = kDim / (kChunkThreads / 64);   // features per wave: 64 or 32
    constexpr int kNt = kFpw / 16;
    const uint32_t li = lane & 15;
    const uint32_t lg = lane >> 4;
    f32x4 o[kNt];
  #pragma unroll
    for (int nt = 0; nt < kNt; ++nt) o[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  #pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t off = li * kPStride + 32 * ks + 8 * lg;   // head li, slots 32 ks + 8 lg ..+8
      const bf16x8 ahi = as_bf16x8(*reinterpret_cast<const u32x4 *>(&phi[off]));
      const bf16x8 alo = as_bf16x8(*reinterpret_cast<const u32x4 *>(&plo[off]));
  #pragma unroll
      for (int nt = 0; nt < kNt; ++nt) {
        // Lane li of group lg receives features n0 + li of slots s0 .. s0+3
        // and s0+4 .. s0+7 (s0 = 32 ks + 8 lg): it addresses slot s0 + li/4
        // (+4), features n0 + 4 (li % 4) .. +4.
        const uint32_t n0 = kFpw * wave + 16 * nt;
        const uint32_t s0 = 32 * ks + 8 * lg;
        const s16x4 b0 = lds_read_tr16(&vt[(s0 + li / 4) * kRowStride + n0 + 4 * (li % 4)]);
        const s16x4 b1 = lds_read_tr16(&vt[(s0 + 4 + li / 4) * kRowStride + n0 + 4 * (li % 4)]);
        const s16x8 b8 = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        const bf16x8 b = __builtin_bit_cast(bf16x8, b8);
        o[nt] = mfma16(ahi, b, o[nt]);
        o[nt] = mfma16(alo, b, o[nt]);
      }
    }
    // D lane l of tile nt: feature kFpw wave + 16 nt + l % 16, heads 4 (l / 16) + i.
    // Non-temporal stores: the chunk outputs are read once, by the combine
    // kernel, from memory; stored as ordinary write-back lines they waited
    // in L2 for the end-of-kernel write-back (8 MiB at 8 rows x 512 slots),
    // which the step then paid for after the last workgroup (34.5 -> 33.8 us
    // per step at 8 rows x 32768 keys).
    float *dst = a.opart + (static_cast<uint64_t>(c) * kHeads + kHg * hg) * kDim;
  #pragma unroll
    for (int nt = 0; nt < kNt; ++nt)
  #pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_nontemporal_store(o[nt][i], &dst[(4 * lg + i) * kDim + kFpw * wave + 16 * nt + li]);
  }
}

}  // namespace ds
