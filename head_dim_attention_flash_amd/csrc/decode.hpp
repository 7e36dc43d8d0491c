// Decode forward (one query row per head): split-KV attention.
//
// Computes the same O = softmax(scale * q K^T + mask) V and lse as the prefill
// kernel for Nq = 1, the "decode" case of the "FFPA Attention Benchmark"
// page. With one query row per head the work is a stream over K and V
// (4 flops per 4 bytes read), so the kernel is bound by HBM bandwidth and
// the dot products run on the vector ALUs: a matrix-core tile would be 31/32
// empty.
//
// Split-KV (flash-decoding): the keys of each (batch, head) are cut into S
// ranges. One wave handles one (batch, query head, range):
//   lane l holds columns 8 (l + 64 j) .. +7 of q (j < ceil(D / 512));
//   per step of 8 keys it loads the 8 K rows and 8 V rows (16 bytes per lane
//   per row, coalesced: a key row is one contiguous 2D-byte run), forms the 8
//   dot products with a butterfly sum across the wave, and updates an online
//   softmax (running max m, sum l, output o rescaled by 2^(m_old - m_new)).
// It writes o / l and m + log2 l (log2 domain) for its range to the
// workspace. The combine kernel then merges the ranges of each head:
//   lse = log2-sum-exp of the range values, O = sum_s 2^(lse_s - lse) o_s.
// Query heads that share a K/V head (GQA) run in neighbouring waves of the
// same XCD, so their K/V reads meet in that L2.
#pragma once

#include "ffpa_common.hpp"

namespace ffpa {

struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;         // may be null
  const void* mask;   // key bias [Nkv] or null
  float* part_o;      // workspace [B * Hq * S, D]
  float* part_lse;    // workspace [B * Hq * S], log2 domain
  int B, Hq, Hkv, Nkv;
  int kv_end;         // keys visible to the row: Nkv, or 1 (top-left causal, row 0)
  int splits;         // S
  int keys_per_split; // multiple of kDecStep
  float scale_log2;
  int n_waves;        // B * Hq * S
  DropParams drop;    // dropout (drop.t = 0: none)
};

constexpr int kDecStep = 8;        // keys per step
constexpr int kDecTargetWaves = 2048;  // 256 CUs x 8 waves (4096 streamed 3 % slower)
constexpr int kDecMinKeys = 256;   // smallest key range worth a wave
constexpr int kDecMaxSplits = 64;

// Number of key ranges per head and keys per range (host and device agree).
__host__ __device__ inline int dec_splits(int B, int Hq, int kv_end) {
  const long heads = (long)B * Hq;
  long s = (kDecTargetWaves + heads - 1) / heads;
  const long cap = (kv_end + kDecMinKeys - 1) / kDecMinKeys;
  if (s > cap) s = cap;
  if (s > kDecMaxSplits) s = kDecMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}
__host__ __device__ inline int dec_keys_per_split(int kv_end, int splits) {
  const int per = (kv_end + splits - 1) / splits;
  return (per + kDecStep - 1) / kDecStep * kDecStep;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Dot product contribution of 8 elements packed as 4 pairs, fp32 accumulate.
template <bool BF16>
__device__ inline float dot8(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(Elem<BF16>::to_f32((uint16_t)(a[e] & 0xffff)), Elem<BF16>::to_f32((uint16_t)(b[e] & 0xffff)), acc);
    acc = fmaf(Elem<BF16>::to_f32((uint16_t)(a[e] >> 16)), Elem<BF16>::to_f32((uint16_t)(b[e] >> 16)), acc);
  }
  return acc;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void dec_split_kernel(DecArgs a) {
  using E = Elem<BF16>;
  using T = typename E::scalar;
  constexpr int GPR = D / 8;                 // 16-byte granules per row
  constexpr int NG = (GPR + 63) / 64;        // granules per lane
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.n_waves) return;              // whole waves leave together
  const int s = wid % a.splits;
  const int bh = wid / a.splits;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int k_lo = s * a.keys_per_split;
  const int k_hi = min(a.kv_end, k_lo + a.keys_per_split);

  bool gok[NG];
  u32x4 qv[NG];
  const T* Q = (const T*)a.q + (size_t)bh * D;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    gok[j] = lane + 64 * j < GPR;
    qv[j] = gok[j] ? *(const u32x4*)(Q + 8 * (lane + 64 * j)) : u32x4{0, 0, 0, 0};
  }
  const T* K = (const T*)a.k + (size_t)(b * a.Hkv + hk) * a.Nkv * D;
  const T* V = (const T*)a.v + (size_t)(b * a.Hkv + hk) * a.Nkv * D;
  const uint16_t* mk = (const uint16_t*)a.mask;

  float m = -INFINITY, l = 0.f;
  float o[NG][8];
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;

  for (int k0 = k_lo; k0 < k_hi; k0 += kDecStep) {
    // K and V are read once (streaming loads, marked non-temporal: 10 % more
    // HBM throughput than plain loads at 16 x 32 heads x 8K keys, D = 512)
    u32x4 kr[kDecStep][NG], vr[kDecStep][NG];
#pragma unroll
    for (int t = 0; t < kDecStep; ++t) {
      const int row = min(k0 + t, k_hi - 1);  // rows past the range: loaded, then masked
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if (gok[j]) {
          kr[t][j] = __builtin_nontemporal_load((const u32x4*)(K + (size_t)row * D + 8 * (lane + 64 * j)));
          vr[t][j] = __builtin_nontemporal_load((const u32x4*)(V + (size_t)row * D + 8 * (lane + 64 * j)));
        } else {
          kr[t][j] = u32x4{0, 0, 0, 0};
          vr[t][j] = u32x4{0, 0, 0, 0};
        }
      }
    }
    float sc[kDecStep];
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < kDecStep; ++t) {
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < NG; ++j) part = dot8<BF16>(qv[j], kr[t][j], part);
      float x = wave_sum(part) * a.scale_log2;
      const int key = k0 + t;
      if (mk != nullptr) x += E::to_f32(mk[min(key, a.Nkv - 1)]) * kLog2e;
      sc[t] = key < k_hi ? x : -INFINITY;
      mt = fmaxf(mt, sc[t]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new == -INFINITY) continue;  // every key so far is masked
    // dropout: the row is query 0; one generator call per 4 keys (the words
    // are the same in every lane)
    uint32_t dw[kDecStep / 4];
    if (a.drop.t != 0) {
#pragma unroll
      for (int c = 0; c < kDecStep / 4; ++c) dw[c] = drop_row_word(a.drop, (int)bh, 0, k0 + 4 * c);
    }
    const float alpha = exp2_fast(m - m_new);  // 0 when m = -inf
    l *= alpha;
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[j][e] *= alpha;
#pragma unroll
    for (int t = 0; t < kDecStep; ++t) {
      const float p0 = exp2_fast(sc[t] - m_new);
      l += p0;
      const float p = (a.drop.t != 0 && !drop_keeps(dw[t / 4], t % 4, a.drop.t)) ? 0.f : p0;
#pragma unroll
      for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[j][2 * e] = fmaf(p, E::to_f32((uint16_t)(vr[t][j][e] & 0xffff)), o[j][2 * e]);
          o[j][2 * e + 1] = fmaf(p, E::to_f32((uint16_t)(vr[t][j][e] >> 16)), o[j][2 * e + 1]);
        }
    }
    m = m_new;
  }

  const float inv = (l > 0.f ? 1.f / l : 0.f) * (a.drop.t != 0 ? a.drop.scale : 1.f);
  float* po = a.part_o + (size_t)wid * D;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    if (!gok[j]) continue;
    f32x4* dst = (f32x4*)(po + 8 * (lane + 64 * j));
    dst[0] = f32x4{o[j][0] * inv, o[j][1] * inv, o[j][2] * inv, o[j][3] * inv};
    dst[1] = f32x4{o[j][4] * inv, o[j][5] * inv, o[j][6] * inv, o[j][7] * inv};
  }
  // v_log_f32 is log2: the range's log-sum-exp in the log2 domain
  if (lane == 0) a.part_lse[wid] = l > 0.f ? m + __builtin_amdgcn_logf(l) : -INFINITY;
}

// One wave per (batch, query head): merge the S ranges.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void dec_combine_kernel(DecArgs a) {
  using E = Elem<BF16>;
  using T = typename E::scalar;
  constexpr int GPR = D / 8;
  constexpr int NG = (GPR + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= a.B * a.Hq) return;
  const float* pl = a.part_lse + (size_t)bh * a.splits;
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, pl[s]);
  float o[NG][8];
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[j][e] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < a.splits; ++s) {
      const float w = exp2_fast(pl[s] - M);
      W += w;
      const float* po = a.part_o + ((size_t)bh * a.splits + s) * D;
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if (lane + 64 * j >= GPR) continue;
        const f32x4 x = *(const f32x4*)(po + 8 * (lane + 64 * j));
        const f32x4 y = *(const f32x4*)(po + 8 * (lane + 64 * j) + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[j][e] = fmaf(w, x[e], o[j][e]);
          o[j][4 + e] = fmaf(w, y[e], o[j][4 + e]);
        }
      }
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  T* O = (T*)a.o + (size_t)bh * D;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    if (lane + 64 * j >= GPR) continue;
    const u32x4 w = {E::pack2(o[j][0] * inv, o[j][1] * inv), E::pack2(o[j][2] * inv, o[j][3] * inv),
                     E::pack2(o[j][4] * inv, o[j][5] * inv), E::pack2(o[j][6] * inv, o[j][7] * inv)};
    *(u32x4*)(O + 8 * (lane + 64 * j)) = w;
  }
  if (a.lse != nullptr && lane == 0)
    a.lse[bh] = W > 0.f ? (M + __builtin_amdgcn_logf(W)) * kLn2 : -INFINITY;
}

template <int D, bool BF16>
hipError_t launch_decode(const DecArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((dec_split_kernel<D, BF16>), dim3((a.n_waves + 3) / 4), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((dec_combine_kernel<D, BF16>), dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
