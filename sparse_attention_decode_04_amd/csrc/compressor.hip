// Learned KV compressor, one decode token per row, on gfx950.
//
// What is computed (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
// kernel deepseek_compressor_rows_bf16; shapes, checks and the one-token
// contract in "mlx-native 0.21.0 src/ops/deepseek_rows.rs",
// dispatch_deepseek_compressor_rows). Each row owns two f32 states (values
// and scores) of coff * ratio rows by P = coff * head_dim features, coff = 2
// for ratio 4 (each window reaches one block back) and 1 otherwise.
//   1. The token at absolute position pos goes to state row
//      slot = (ratio if overlapping else 0) + pos % ratio: the value itself
//      (0 if not finite) and its score plus the position embedding of
//      pos % ratio (NaN if that sum or the value is not finite).
//   2. If pos + 1 ends a block, feature f < head_dim of the output pools the
//      window: with overlap, state rows [0, ratio) at feature f (the previous
//      block) and rows [ratio, 2 ratio) at feature head_dim + f (this block);
//      otherwise rows [0, ratio) at feature f. The pooled value is
//      sum_i e^(s_i - m) v_i / sum_i e^(s_i - m), m = max_i s_i, rounded to
//      bf16. A NaN or +inf window score, a non-finite window value, a
//      non-finite pooled value or RMS scale element makes the row invalid.
//      Then out = bf16(c * rsqrt(mean(c^2) + eps) * norm), or zeros for an
//      invalid row or a non-finite result. With overlap the current block
//      then becomes the previous one (rows [0, ratio) <- rows [ratio, 2 ratio)).
//      A token that does not end a block writes a zero output.
//
// Layout of the work: one workgroup per row, launched on XCD r (block
// b -> XCD b % 8). Lane = feature within a 64-feature group; the waves share
// out the window items (ratio 4: 4 waves, wave w owns items w and w + 4 of
// every group) or items and groups (ratio 128: 16 waves, wave w owns group
// w / 2 and items w % 2, w % 2 + 2, ...). Every state element a thread reads
// or writes lies in its own features and its own item rows (with overlap
// wave w also shifts row w from row w + 4, and the token's row ratio + t is
// wave t's), so the state needs no synchronisation between threads, and all
// of a thread's stores follow its loads. Each thread keeps an online max /
// sum / weighted sum over its items, streaming the 128-item windows in
// batches of 8 with the next batch in flight; the item-sharing waves'
// partials meet in LDS, where each feature is pooled, rounded, summed for
// the RMS scale and normalised.
#include "device_common.hpp"
#include "ds_rows_internal.hpp"

namespace ds {

template <int kHd, int kRatio>
struct CompShape {
  static constexpr bool kOverlap = kRatio == 4;
  static constexpr int kP = (kOverlap ? 2 : 1) * kHd;
  static constexpr int kWindow = kOverlap ? 2 * kRatio : kRatio;
  static constexpr int kThreads = kOverlap ? 256 : 1024;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kGroups = kHd / 64;                       // 64-feature groups
  static constexpr int kGroupWays = kOverlap ? 1 : kGroups;      // waves sharing out the groups
  static constexpr int kItemWays = kWaves / kGroupWays;          // waves sharing out the items
  static constexpr int kMyGroups = kGroups / kGroupWays;         // groups per thread
  static constexpr int kMyItems = kWindow / kItemWays;           // items per thread
  static constexpr int kBatch = kMyItems < 8 ? kMyItems : 8;     // items per load batch
  static constexpr int kBatches = kMyItems / kBatch;
  static constexpr int kPer = (kHd + kThreads - 1) / kThreads;   // features per thread when combining
  static_assert(kWaves % kGroupWays == 0 && kWindow % kItemWays == 0 && kMyItems % kBatch == 0, "split");
  static_assert(!kOverlap || kItemWays == kRatio, "overlap: wave w owns items w and w + ratio");
};

__device__ __forceinline__ float bf16_round(float x) {
  return static_cast<float>(static_cast<__bf16>(x));
}
__device__ __forceinline__ bool finitef(float x) { return __builtin_isfinite(x); }

__device__ __forceinline__ void sanitize(float vi, float si, float &v, float &s) {
  v = finitef(vi) ? vi : 0.0f;
  s = (finitef(si) && finitef(vi)) ? si : __builtin_nanf("");
}

template <int kHd, int kRatio>
__global__ __launch_bounds__((CompShape<kHd, kRatio>::kThreads)) void compressor_kernel(CompressorArgs a) {
  using S = CompShape<kHd, kRatio>;
  constexpr bool overlap = S::kOverlap;
  constexpr uint32_t P = S::kP, hd = kHd, ratio = kRatio;
  const uint32_t r = blockIdx.x;
  // The row's arguments in one batch of scalar loads, waited for once (read
  // one after another they would cost dependent round trips).
  uint32_t rows = a.rows, pos = a.start_pos[r];
  uint64_t kvs_bits = reinterpret_cast<uint64_t>(a.kv_state[r]), scs_bits = reinterpret_cast<uint64_t>(a.score_state[r]);
  uint64_t kv_bits = reinterpret_cast<uint64_t>(a.kv), sc_bits = reinterpret_cast<uint64_t>(a.score);
  uint64_t ape_bits = reinterpret_cast<uint64_t>(a.ape), out_bits = reinterpret_cast<uint64_t>(a.out);
  asm volatile("" : "+s"(rows), "+s"(pos), "+s"(kvs_bits), "+s"(scs_bits), "+s"(kv_bits), "+s"(sc_bits), "+s"(ape_bits),
               "+s"(out_bits));
  if (r >= rows) return;
  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t iw = wave % S::kItemWays;                        // item way
  const uint32_t g0 = (wave / S::kItemWays) * S::kMyGroups;       // first group of this thread
  const uint32_t token = pos % ratio;
  const uint32_t slot = (overlap ? ratio : 0) + token;
  const bool emit = (pos + 1) % ratio == 0;
  float *kvs = global_ptr<float>(kvs_bits);
  float *scs = global_ptr<float>(scs_bits);
  const float *kin = global_ptr<const float>(kv_bits) + static_cast<uint64_t>(r) * P;
  const float *scin = global_ptr<const float>(sc_bits) + static_cast<uint64_t>(r) * P;
  const float *ape = global_ptr<const float>(ape_bits) + static_cast<uint64_t>(token) * P;
  uint16_t *out = global_ptr<uint16_t>(out_bits) + static_cast<uint64_t>(r) * hd;
  const bool owns_slot = iw == slot % S::kItemWays;               // this thread's items include the slot

  // The token at features f and head_dim + f of each of this thread's groups.
  float tv[S::kMyGroups][2], ts[S::kMyGroups][2];
#pragma unroll
  for (int g = 0; g < S::kMyGroups; ++g) {
    const uint32_t f = 64 * (g0 + g) + lane;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t x = (overlap && h == 1) ? hd + f : f;
      tv[g][h] = kin[x];
      ts[g][h] = scin[x] + ape[x];
    }
  }

  if (!emit) {
    if (owns_slot) {
#pragma unroll
      for (int g = 0; g < S::kMyGroups; ++g) {
        const uint32_t f = 64 * (g0 + g) + lane;
#pragma unroll
        for (int h = 0; h < (overlap ? 2 : 1); ++h) {
          float v, sc;
          sanitize(tv[g][h], ts[g][h], v, sc);
          kvs[slot * P + h * hd + f] = v;
          scs[slot * P + h * hd + f] = sc;
        }
      }
    }
    for (uint32_t f = tid; f < hd; f += S::kThreads) out[f] = 0;
    return;
  }

  __shared__ float pm[S::kItemWays][kHd];
  __shared__ float pd[S::kItemWays][kHd];
  __shared__ float pn[S::kItemWays][kHd];
  __shared__ float red[S::kWaves];
  __shared__ uint32_t sh_bad;
  if (tid == 0) sh_bad = 0;

  // RMS scale of the features this thread combines (j = tid + threads * e).
  float nrm[S::kPer];
#pragma unroll
  for (int e = 0; e < S::kPer; ++e) nrm[e] = a.norm[min(tid + S::kThreads * e, hd - 1)];
  // Overlap: row wave + 4 at feature f (the shift's source; item w + 4 is
  // read at head_dim + f).
  float shift_v[S::kMyGroups], shift_s[S::kMyGroups];
  if constexpr (overlap) {
#pragma unroll
    for (int g = 0; g < S::kMyGroups; ++g) {
      const uint32_t f = 64 * (g0 + g) + lane;
      shift_v[g] = kvs[(iw + ratio) * P + f];
      shift_s[g] = scs[(iw + ratio) * P + f];
    }
  }
  // Item k of this thread is state row iw + kItemWays * k; batches of
  // kBatch items alternate between two register buffers.
  using Buf = float[S::kMyGroups][S::kBatch];
  Buf sb0, vb0, sb1, vb1;
  auto load_batch = [&](int b, Buf &sbb, Buf &vbb) {
#pragma unroll
    for (int g = 0; g < S::kMyGroups; ++g) {
      const uint32_t f = 64 * (g0 + g) + lane;
#pragma unroll
      for (int q = 0; q < S::kBatch; ++q) {
        const uint32_t i = iw + S::kItemWays * (b * S::kBatch + q);
        const uint32_t x = (overlap && i >= ratio) ? hd + f : f;
        sbb[g][q] = scs[i * P + x];
        vbb[g][q] = kvs[i * P + x];
      }
    }
  };
  float m[S::kMyGroups], den[S::kMyGroups], num[S::kMyGroups];
  float last_v[S::kMyGroups], last_s[S::kMyGroups];   // overlap: item iw + 4 (this block, head_dim + f)
#pragma unroll
  for (int g = 0; g < S::kMyGroups; ++g) { m[g] = -__builtin_inff(); den[g] = 0.0f; num[g] = 0.0f; }
  bool bad = false;
  auto process = [&](int b, Buf &sbb, Buf &vbb) {
#pragma unroll
    for (int g = 0; g < S::kMyGroups; ++g) {
      // The token's values replace its slot.
#pragma unroll
      for (int q = 0; q < S::kBatch; ++q) {
        const uint32_t i = iw + S::kItemWays * (b * S::kBatch + q);
        if (i == slot) sanitize(tv[g][overlap ? 1 : 0], ts[g][overlap ? 1 : 0], vbb[g][q], sbb[g][q]);
      }
      float mb = m[g];
#pragma unroll
      for (int q = 0; q < S::kBatch; ++q) {
        bad |= __builtin_isnan(sbb[g][q]) || sbb[g][q] == __builtin_inff() || !finitef(vbb[g][q]);
        mb = fmaxf(mb, sbb[g][q]);
      }
      if (mb != -__builtin_inff()) {
        if (m[g] != -__builtin_inff()) {
          const float sc = __expf(m[g] - mb);
          den[g] *= sc;
          num[g] *= sc;
        }
#pragma unroll
        for (int q = 0; q < S::kBatch; ++q) {
          const float w = __expf(sbb[g][q] - mb);
          den[g] += w;
          num[g] = fmaf(w, vbb[g][q], num[g]);
        }
        m[g] = mb;
      }
      if constexpr (overlap) {
        last_v[g] = vbb[g][1];
        last_s[g] = sbb[g][1];
      }
    }
  };
  load_batch(0, sb0, vb0);
  if constexpr (S::kBatches == 1) {
    process(0, sb0, vb0);
  } else {
    static_assert(S::kBatches % 2 == 0, "batches go in pairs");
#pragma unroll 1
    for (int b = 0; b < S::kBatches; b += 2) {
      // Loads are unconditional: past the end, the last batch is loaded
      // again (from cache) and not used.
      load_batch(b + 1, sb1, vb1);
      process(b, sb0, vb0);
      load_batch(min(b + 2, S::kBatches - 1), sb0, vb0);
      process(b + 1, sb1, vb1);
    }
  }
#pragma unroll
  for (int g = 0; g < S::kMyGroups; ++g) {
    const uint32_t j = 64 * (g0 + g) + lane;
    pm[iw][j] = m[g];
    pd[iw][j] = den[g];
    pn[iw][j] = num[g];
  }
  // State stores (after this thread's loads): the token's row, then with
  // overlap row w <- row w + 4 (both halves).
#pragma unroll
  for (int g = 0; g < S::kMyGroups; ++g) {
    const uint32_t f = 64 * (g0 + g) + lane;
    if constexpr (overlap) {
      if (iw + ratio == slot) sanitize(tv[g][0], ts[g][0], shift_v[g], shift_s[g]);
      if (owns_slot) {
        kvs[slot * P + f] = shift_v[g];
        scs[slot * P + f] = shift_s[g];
        kvs[slot * P + hd + f] = last_v[g];
        scs[slot * P + hd + f] = last_s[g];
      }
      kvs[iw * P + f] = shift_v[g];
      scs[iw * P + f] = shift_s[g];
      kvs[iw * P + hd + f] = last_v[g];
      scs[iw * P + hd + f] = last_s[g];
    } else {
      if (owns_slot) {
        float v, sc;
        sanitize(tv[g][0], ts[g][0], v, sc);
        kvs[slot * P + f] = v;
        scs[slot * P + f] = sc;
      }
    }
  }
  if (__ballot(bad) != 0 && lane == 0) atomicOr(&sh_bad, 1u);
  __syncthreads();

  // Per feature j = tid + threads * e: pool across the item ways, round to
  // bf16, and sum the squares for the RMS scale.
  float c[S::kPer];
  bool cbad = false;
  float sq = 0.0f;
#pragma unroll
  for (int e = 0; e < S::kPer; ++e) {
    const uint32_t j = tid + S::kThreads * e;
    c[e] = 0.0f;
    if (j < hd) {
      float mm = pm[0][j];
#pragma unroll
      for (int w = 1; w < S::kItemWays; ++w) mm = fmaxf(mm, pm[w][j]);
      float dd = 0.0f, nn = 0.0f;
      if (mm != -__builtin_inff()) {
#pragma unroll
        for (int w = 0; w < S::kItemWays; ++w) {
          if (pm[w][j] != -__builtin_inff()) {
            const float sc = __expf(pm[w][j] - mm);
            dd = fmaf(pd[w][j], sc, dd);
            nn = fmaf(pn[w][j], sc, nn);
          }
        }
      }
      const float pooled = nn / dd;
      const bool fin = finitef(pooled);
      c[e] = bf16_round(fin ? pooled : 0.0f);
      cbad |= !fin || !finitef(nrm[e]);
      sq = fmaf(c[e], c[e], sq);
    }
  }
  if (__ballot(cbad) != 0 && lane == 0) atomicOr(&sh_bad, 1u);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o);
  if (lane == 0) red[wave] = sq;
  __syncthreads();
  float total = 0.0f;
#pragma unroll
  for (int w = 0; w < S::kWaves; ++w) total += red[w];
  bool row_bad = sh_bad != 0 || !finitef(total);
  const float rms = row_bad ? 0.0f : 1.0f / sqrtf(total / static_cast<float>(hd) + a.eps);
  row_bad |= !finitef(rms);
  float y[S::kPer];
  bool ybad = false;
#pragma unroll
  for (int e = 0; e < S::kPer; ++e) {
    y[e] = c[e] * rms * nrm[e];
    ybad |= tid + S::kThreads * e < hd && !finitef(y[e]);
  }
  __syncthreads();
  if (__ballot(ybad) != 0 && lane == 0) atomicOr(&sh_bad, 2u);
  __syncthreads();
  row_bad |= (sh_bad & 2u) != 0;
#pragma unroll
  for (int e = 0; e < S::kPer; ++e) {
    const uint32_t j = tid + S::kThreads * e;
    if (j < hd) out[j] = row_bad ? 0 : __builtin_bit_cast(uint16_t, static_cast<__bf16>(y[e]));
  }
}

hipError_t launch_compressor(const CompressorArgs &a, hipStream_t s) {
  const dim3 grid(a.rows);
  if (a.ratio == 4 && a.head_dim == 128)
    hipLaunchKernelGGL((compressor_kernel<128, 4>), grid, dim3(CompShape<128, 4>::kThreads), 0, s, a);
  else if (a.ratio == 4 && a.head_dim == 512)
    hipLaunchKernelGGL((compressor_kernel<512, 4>), grid, dim3(CompShape<512, 4>::kThreads), 0, s, a);
  else if (a.ratio == 128 && a.head_dim == 512)
    hipLaunchKernelGGL((compressor_kernel<512, 128>), grid, dim3(CompShape<512, 128>::kThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ds
