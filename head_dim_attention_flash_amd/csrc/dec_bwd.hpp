// Backward of the decode case (one query row per head): dQ, dK, dV.
//
// The gradient of the attention of "naive_math" (section 3 of the
// attention-kernel-profiler design document) for Nq = 1, the "decode" case of
// the "FFPA Attention Benchmark" page, with the backward conventions of the
// "Backward Pass" tables of "More Benchmark". For the single row of head h:
//   s_k   = scale q . K_k + mask_k,   P_k = exp(s_k - lse)  (lse from the forward)
//   dP_k  = dO . V_k,                 delta = dO . O,   dS_k = P_k (dP_k - delta)
//   dV_k  = sum over the group's query heads of P_k dO
//   dK_k  = scale * sum over the group's query heads of dS_k q
//   dQ    = scale * sum_k dS_k K_k
// With one row per head every key is touched once: 4 flops per 4 bytes of K
// and V read and dK and dV written, so the pass is bound by HBM, and the dot
// products run on the vector ALUs (a matrix-core tile would be 31/32 empty).
//
// One wave handles one (batch, kv head, key range) for all G query heads of
// the group, so each key's dK and dV are written once, by one wave:
//   lane l holds columns 8 (l + 64 j) .. +7 (j < ceil(D / 512)) of q, dO and
//   of the fp32 dQ partial of each query head;
//   per step of 8 keys it loads the 8 K rows and 8 V rows (16 bytes per lane
//   per row, coalesced; up to D = 512 one step ahead), forms 2 G dot products
//   per key with butterfly sums across the wave, and writes the 8 dK and dV
//   rows.
// dQ is a sum over all keys: each wave writes its range's partial (fp32) to
// the workspace and a second kernel adds the ranges of each head in range
// order (deterministic) and rounds once.
#pragma once

#include "ffpa_common.hpp"
#include "decode.hpp"

namespace ffpa {

struct DecBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;   // natural log, [B * Hq]; -inf for a row that sees no key
  const void* mask;   // the row's additive mask [Nkv] (key bias or the one query row) or null
  void* dq;
  void* dk;
  void* dv;
  float* part_dq;     // workspace [B * Hkv * S, G, D] (fp32)
  int B, Hq, Hkv, Nkv;
  int kv_end;         // keys the row sees: Nkv, or 1 (causal, top-left: row 0 sees key 0)
  int splits;         // S key ranges per (batch, kv head); together they cover all Nkv keys
  int keys_per_split; // multiple of kDecStep
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  int n_waves;        // B * Hkv * S
};

// Key ranges per (batch, kv head) (host and device agree): about
// kDecBwdTargetWaves waves in all (4096 and 8192 measured 1 % slower at B16
// H32 Nkv 8192 D 512), ranges of at least kDecMinKeys keys, at most
// kDecMaxSplits per kv head.
constexpr int kDecBwdTargetWaves = 2048;
__host__ __device__ inline int dec_bwd_splits(int B, int Hkv, int Nkv) {
  const long heads = (long)B * Hkv;
  long s = (kDecBwdTargetWaves + heads - 1) / heads;
  const long cap = (Nkv + kDecMinKeys - 1) / kDecMinKeys;
  if (s > cap) s = cap;
  if (s > kDecMaxSplits) s = kDecMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

// Workspace bytes of the decode backward: the fp32 dQ partial of every range
// of every query head.
__host__ inline size_t dec_bwd_bytes(int B, int Hq, int Hkv, int Nkv, int D) {
  return (size_t)B * Hq * (size_t)dec_bwd_splits(B, Hkv, Nkv) * D * sizeof(float);
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void dec_bwd_kernel(DecBwdArgs a) {
  using E = Elem<BF16>;
  using T = typename E::scalar;
  constexpr int GPR = D / 8;           // 16-byte granules per row
  constexpr int NG = (GPR + 63) / 64;  // granules per lane
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= a.n_waves) return;  // whole waves leave together
  const int s = wid % a.splits;
  const int bk = wid / a.splits;  // b * Hkv + hk
  const int b = bk / a.Hkv, hk = bk % a.Hkv;
  const int k_lo = s * a.keys_per_split;
  const int k_hi = min(a.Nkv, k_lo + a.keys_per_split);

  bool gok[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) gok[j] = lane + 64 * j < GPR;
  auto row_load = [&](const T* base, int j) {
    return gok[j] ? *(const u32x4*)(base + 8 * (lane + 64 * j)) : u32x4{0, 0, 0, 0};
  };

  // the group's query rows: q, dO, delta = dO . O and lse in the log2 domain
  // (+inf for a row that sees no key, so that every P of it is 0)
  u32x4 qv[G][NG], dov[G][NG];
  float delta[G], lse2[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t bh = (size_t)b * a.Hq + (size_t)hk * G + h;
    const T* Qr = (const T*)a.q + bh * D;
    const T* Or = (const T*)a.o + bh * D;
    const T* Dr = (const T*)a.dout + bh * D;
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      qv[h][j] = row_load(Qr, j);
      dov[h][j] = row_load(Dr, j);
      part = dot8<BF16>(dov[h][j], row_load(Or, j), part);
    }
    delta[h] = wave_sum(part);
    const float l = a.lse[bh];
    lse2[h] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
  const T* K = (const T*)a.k + (size_t)bk * a.Nkv * D;
  const T* V = (const T*)a.v + (size_t)bk * a.Nkv * D;
  T* dK = (T*)a.dk + (size_t)bk * a.Nkv * D;
  T* dV = (T*)a.dv + (size_t)bk * a.Nkv * D;
  const uint16_t* mk = (const uint16_t*)a.mask;

  float dq[G][NG][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) dq[h][j][e] = 0.f;

  // K and V are read once (streaming loads); rows past the range are loaded
  // from the last row, then neither used nor written. Up to D = 512 the loads
  // run one step of 8 keys ahead (2.5 % faster at B16 H32 Nkv 8192 D 512; the
  // registers that costs would halve the waves per SIMD above 512).
  constexpr bool kAhead = NG == 1;
  u32x4 kn[kDecStep][NG], vn[kDecStep][NG];
  auto load_step = [&](int k0) {
#pragma unroll
    for (int t = 0; t < kDecStep; ++t) {
      const int row = min(k0 + t, k_hi - 1);
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if (gok[j]) {
          kn[t][j] = __builtin_nontemporal_load((const u32x4*)(K + (size_t)row * D + 8 * (lane + 64 * j)));
          vn[t][j] = __builtin_nontemporal_load((const u32x4*)(V + (size_t)row * D + 8 * (lane + 64 * j)));
        } else {
          kn[t][j] = u32x4{0, 0, 0, 0};
          vn[t][j] = u32x4{0, 0, 0, 0};
        }
      }
    }
  };
  if (kAhead && k_lo < k_hi) load_step(k_lo);
  for (int k0 = k_lo; k0 < k_hi; k0 += kDecStep) {
    if (!kAhead) load_step(k0);
    u32x4 kr[kDecStep][NG], vr[kDecStep][NG];
#pragma unroll
    for (int t = 0; t < kDecStep; ++t)
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        kr[t][j] = kn[t][j];
        vr[t][j] = vn[t][j];
      }
    if (kAhead && k0 + kDecStep < k_hi) load_step(k0 + kDecStep);
    // P and dS of the 8 keys for every query head of the group
    float p[kDecStep][G], ds[kDecStep][G];
#pragma unroll
    for (int t = 0; t < kDecStep; ++t) {
      const int key = k0 + t;
      const float bias = (mk != nullptr) ? E::to_f32(mk[min(key, a.Nkv - 1)]) * kLog2e : 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float ps = 0.f, pd = 0.f;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
          ps = dot8<BF16>(qv[h][j], kr[t][j], ps);
          pd = dot8<BF16>(dov[h][j], vr[t][j], pd);
        }
        const float x = wave_sum(ps) * a.scale_log2 + bias;
        const float dp = wave_sum(pd);
        const float pk = key < a.kv_end ? exp2_fast(x - lse2[h]) : 0.f;
        p[t][h] = pk;
        ds[t][h] = pk * (dp - delta[h]);
      }
    }
    // dV_k = sum_h P dO, dK_k = scale sum_h dS q (one rounding each);
    // dQ_h += dS K_k
#pragma unroll
    for (int t = 0; t < kDecStep; ++t) {
      const int key = k0 + t;
      if (key >= k_hi) break;  // wave-uniform
#pragma unroll
      for (int j = 0; j < NG; ++j) {
        if (!gok[j]) continue;
        float dvx[8], dkx[8], kx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[2 * e] = E::to_f32((uint16_t)(kr[t][j][e] & 0xffff));
          kx[2 * e + 1] = E::to_f32((uint16_t)(kr[t][j][e] >> 16));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) dvx[e] = dkx[e] = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d0 = E::to_f32((uint16_t)(dov[h][j][e] & 0xffff));
            const float d1 = E::to_f32((uint16_t)(dov[h][j][e] >> 16));
            const float q0 = E::to_f32((uint16_t)(qv[h][j][e] & 0xffff));
            const float q1 = E::to_f32((uint16_t)(qv[h][j][e] >> 16));
            dvx[2 * e] = fmaf(p[t][h], d0, dvx[2 * e]);
            dvx[2 * e + 1] = fmaf(p[t][h], d1, dvx[2 * e + 1]);
            dkx[2 * e] = fmaf(ds[t][h], q0, dkx[2 * e]);
            dkx[2 * e + 1] = fmaf(ds[t][h], q1, dkx[2 * e + 1]);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) dq[h][j][e] = fmaf(ds[t][h], kx[e], dq[h][j][e]);
        }
        const u32x4 wv = {E::pack2(dvx[0], dvx[1]), E::pack2(dvx[2], dvx[3]), E::pack2(dvx[4], dvx[5]),
                          E::pack2(dvx[6], dvx[7])};
        const u32x4 wk = {E::pack2(a.scale * dkx[0], a.scale * dkx[1]), E::pack2(a.scale * dkx[2], a.scale * dkx[3]),
                          E::pack2(a.scale * dkx[4], a.scale * dkx[5]), E::pack2(a.scale * dkx[6], a.scale * dkx[7])};
        __builtin_nontemporal_store(wv, (u32x4*)(dV + (size_t)key * D + 8 * (lane + 64 * j)));
        __builtin_nontemporal_store(wk, (u32x4*)(dK + (size_t)key * D + 8 * (lane + 64 * j)));
      }
    }
  }

  // this range's scale * sum_k dS_k K_k of each query head
  float* pq = a.part_dq + (size_t)wid * G * D;
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      if (!gok[j]) continue;
      f32x4* dst = (f32x4*)(pq + (size_t)h * D + 8 * (lane + 64 * j));
      dst[0] = f32x4{a.scale * dq[h][j][0], a.scale * dq[h][j][1], a.scale * dq[h][j][2], a.scale * dq[h][j][3]};
      dst[1] = f32x4{a.scale * dq[h][j][4], a.scale * dq[h][j][5], a.scale * dq[h][j][6], a.scale * dq[h][j][7]};
    }
}

// One wave per (batch, query head): dQ = the sum of its ranges' partials, in
// range order.
template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void dec_bwd_combine_kernel(DecBwdArgs a) {
  using E = Elem<BF16>;
  using T = typename E::scalar;
  constexpr int GPR = D / 8;
  constexpr int NG = (GPR + 63) / 64;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq, hq = bh % a.Hq;
  const int hk = hq / G, h = hq % G;
  float acc[NG][8];
#pragma unroll
  for (int j = 0; j < NG; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* pq = a.part_dq + (((size_t)(b * a.Hkv + hk) * a.splits + s) * G + h) * D;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      if (lane + 64 * j >= GPR) continue;
      const f32x4 x = *(const f32x4*)(pq + 8 * (lane + 64 * j));
      const f32x4 y = *(const f32x4*)(pq + 8 * (lane + 64 * j) + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[j][e] += x[e];
        acc[j][4 + e] += y[e];
      }
    }
  }
  T* dQ = (T*)a.dq + (size_t)bh * D;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    if (lane + 64 * j >= GPR) continue;
    const u32x4 w = {E::pack2(acc[j][0], acc[j][1]), E::pack2(acc[j][2], acc[j][3]),
                     E::pack2(acc[j][4], acc[j][5]), E::pack2(acc[j][6], acc[j][7])};
    *(u32x4*)(dQ + 8 * (lane + 64 * j)) = w;
  }
}

// Host launcher: the range kernel, then the combine. The caller has checked
// Hq == G * Hkv and the sizes of the workspace and grids.
template <int D, bool BF16, int G>
hipError_t launch_dec_bwd(const DecBwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((dec_bwd_kernel<D, BF16, G>), dim3((a.n_waves + 3) / 4), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((dec_bwd_combine_kernel<D, BF16, G>), dim3((a.B * a.Hq + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
