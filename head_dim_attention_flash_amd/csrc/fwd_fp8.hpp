// FP8 forward: S = Q K^T and O = P V on the gfx950 fp8 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4, OCP e4m3 operands, fp32 accumulation), for
// Nq > 1 and D a multiple of 64 in [128, 512]. The pages list FP8 attention
// kernels beside the 16-bit ones ("FFPA Attention Benchmark", "FP8 and FP4"),
// without their quantisation; the scheme here is the plainest one:
//  - Q, K and V of each head are quantised with one scale per head and tensor:
//    x8 = e4m3(x * (448 / amax)), amax = max |x| over the head (a 448-sized
//    code is e4m3's largest finite value), rounded to nearest even;
//  - P = 2^(s - m) is quantised as e4m3(64 P) against a running reference
//    m per row: over the keys in tiles of 64, m rises to a tile's maximum
//    score when that exceeds m by more than 2.5 (log2 units), and only then
//    (so P <= 2^2.5 and 64 P < 448); the row sum l takes the unquantised P.
//    The loose threshold keeps the O rescales rare (on N(0, 1) scores about
//    one row in 100 rises after its first tile); 64 P keeps P >= 2^-12 in
//    e4m3's normal range;
//  - O = (sum_j P8_j V8_j) * (amax_V / 448) / (64 l), in fp32, then rounded
//    to the 16-bit output type; lse as for the 16-bit kernels.
// A pre-pass writes the quantised tensors into the workspace: Q8, K8 row-major
// and V8 transposed per 64-key tile with the keys of a tile permuted (see
// f8_key_of_pos) so that each lane's MFMA operand is 32 contiguous bytes.
#pragma once

#include "ffpa_common.hpp"

namespace ffpa {

typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8Rows = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kF8Bc = 64;     // keys per staged tile
constexpr float kF8Max = 448.f;
constexpr float kF8PScale = 64.f;
constexpr float kF8PLog2 = 6.f;  // log2 of the P scale
constexpr float kF8Tau = 2.5f;  // rescale threshold (log2 units)

struct Fp8Args {
  const void* q;  // the 16-bit inputs (pre-pass)
  const void* k;
  const void* v;
  uint8_t* q8;    // workspace: [B, Hq, Nq, D] e4m3
  uint8_t* k8;    // [B, Hkv, Nkv, D]
  uint8_t* vt8;   // [B, Hkv, nkt, D, 64]: tile t, row d, position p -> key 64 t + f8_key_of_pos(p)
  float* amax;    // [3][B * Hq]: max |x| per head of Q (0), K (1), V (2); K and V use B * Hkv
  void* o;
  float* lse;     // nullable
  int B, Hq, Hkv, Nq, Nkv;
  int causal;
  float scale_log2;  // softmax scale * log2(e)
  int nkt;           // ceil(Nkv / 64)
  int n_qtiles;      // ceil(Nq / 128)
  int total_wg;
};

// Position p (0 .. 63) of a V^T tile row -> key within the tile. Lane half h
// of the P V product holds positions 32 h .. 32 h + 31; position 32 h + j is
// score register j % 16 of key block j / 16 of that half: key 32 (j / 16) +
// 8 ((j % 16) / 4) + 4 h + j % 4, the row layout of a 32x32 MFMA result.
__host__ __device__ inline int f8_key_of_pos(int p) {
  const int h = p >> 5, j = p & 31;
  return 32 * (j >> 4) + 8 * ((j & 15) >> 2) + 4 * h + (j & 3);
}

// Dequantisation factor amax / 448 of a head (0 for an all-zero head).
__device__ inline float f8_descale(float amax) { return amax / kF8Max; }
// Quantisation factor 448 / amax (1 for an all-zero head: every code is 0).
__device__ inline float f8_qscale(float amax) { return amax > 0.f ? kF8Max / amax : 1.f; }

// Four e4m3 codes of four floats (round to nearest even), bytes in order.
__device__ inline uint32_t f8_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// ---------------------------------------------------------------------------
// Pre-pass.
// ---------------------------------------------------------------------------
// (a template only so that every file including this header has its own instance)
template <int D>
__global__ __launch_bounds__(256) void f8_zero_kernel(float* amax, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) amax[i] = 0.f;
}

// max |x| per head: workgroup (t, head, slab of kF8AmaxRows rows) of tensor t
// (0 Q, 1 K, 2 V), four 16-byte loads in flight per thread; the workgroup's
// max goes to the head's slot with one atomicMax on the bits (non-negative
// floats order as their bit patterns). Slabs of 256 rows keep the atomics to
// one per 256 rows: thousands of them on a few cache lines would serialise.
constexpr int kF8AmaxRows = 256;
template <int D, bool BF16>
__global__ __launch_bounds__(256) void f8_amax_kernel(Fp8Args a) {
  using E = Elem<BF16>;
  __shared__ float wmax[4];
  const int nq_slabs = (a.Nq + kF8AmaxRows - 1) / kF8AmaxRows, nk_slabs = (a.Nkv + kF8AmaxRows - 1) / kF8AmaxRows;
  const int q_wg = a.B * a.Hq * nq_slabs, k_wg = a.B * a.Hkv * nk_slabs;
  int w = blockIdx.x, t = 0;
  if (w >= q_wg) {
    w -= q_wg;
    t = w >= k_wg ? 2 : 1;
    if (t == 2) w -= k_wg;
  }
  const int slabs = t == 0 ? nq_slabs : nk_slabs, rows = t == 0 ? a.Nq : a.Nkv;
  const int head = w / slabs, slab = w % slabs;
  const uint16_t* x = (const uint16_t*)(t == 0 ? a.q : t == 1 ? a.k : a.v) + (size_t)head * rows * D;
  const int r0 = slab * kF8AmaxRows, r1 = min(rows, r0 + kF8AmaxRows);
  const int n8 = (r1 - r0) * D / 8;
  const uint16_t* x0 = x + (size_t)r0 * D;
  float m = 0.f;
  auto fold = [&](const u32x4& g) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m = fmaxf(m, fabsf(E::to_f32((uint16_t)(g[e] & 0xffff))));
      m = fmaxf(m, fabsf(E::to_f32((uint16_t)(g[e] >> 16))));
    }
  };
  int i = threadIdx.x;
  for (; i + 3 * 256 < n8; i += 4 * 256) {
    u32x4 g[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) g[u] = *(const u32x4*)(x0 + 8 * (i + 256 * u));
#pragma unroll
    for (int u = 0; u < 4; ++u) fold(g[u]);
  }
  for (; i < n8; i += 256) fold(*(const u32x4*)(x0 + 8 * i));
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const int base = t == 0 ? 0 : t == 1 ? a.B * a.Hq : a.B * a.Hq + a.B * a.Hkv;
    atomicMax((unsigned int*)(a.amax + base + head), __float_as_uint(m));
  }
}

// Q8 and K8: 16 elements (one 16-byte output) per thread.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void f8_quant_qk_kernel(Fp8Args a) {
  using E = Elem<BF16>;
  const int64_t nq = (int64_t)a.B * a.Hq * a.Nq * (D / 16), nk = (int64_t)a.B * a.Hkv * a.Nkv * (D / 16);
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nq + nk) return;
  const bool is_q = i < nq;
  if (!is_q) i -= nq;
  const int64_t row = i / (D / 16);
  const int head = (int)(row / (is_q ? a.Nq : a.Nkv));
  const float s = f8_qscale(a.amax[(is_q ? 0 : a.B * a.Hq) + head]);
  const uint16_t* x = (const uint16_t*)(is_q ? a.q : a.k) + 16 * i;
  const u32x4 g0 = *(const u32x4*)x, g1 = *(const u32x4*)(x + 8);
  auto lo = [&](uint32_t w) { return E::to_f32((uint16_t)(w & 0xffff)) * s; };
  auto hi = [&](uint32_t w) { return E::to_f32((uint16_t)(w >> 16)) * s; };
  u32x4 out;
  out[0] = f8_pack4(lo(g0[0]), hi(g0[0]), lo(g0[1]), hi(g0[1]));
  out[1] = f8_pack4(lo(g0[2]), hi(g0[2]), lo(g0[3]), hi(g0[3]));
  out[2] = f8_pack4(lo(g1[0]), hi(g1[0]), lo(g1[1]), hi(g1[1]));
  out[3] = f8_pack4(lo(g1[2]), hi(g1[2]), lo(g1[3]), hi(g1[3]));
  *(u32x4*)((is_q ? a.q8 : a.k8) + 16 * i) = out;
}

// V8^T: workgroup per (kv head, tile of 64 keys); the tile's 16-bit rows go
// through LDS (64 x D), then each thread writes 16 positions of two V^T rows.
// Keys at or past Nkv are written as 0.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void f8_quant_vt_kernel(Fp8Args a) {
  using E = Elem<BF16>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  // the tile [64 keys][D], 16-byte granule g of key row r stored at granule
  // g ^ swz(r): the four rows a wave reads at once (keys r, r + 4, r + 32,
  // r + 36 of the position order) then sit in distinct 32-byte bank windows
  char* tile = smem_raw;
  auto swz = [](int r) { return 2 * (((r >> 2) & 1) | (((r >> 5) & 1) << 1)); };
  const int head = blockIdx.x / a.nkt, kt = blockIdx.x % a.nkt;
  const uint16_t* v = (const uint16_t*)a.v + ((size_t)head * a.Nkv + (size_t)kt * kF8Bc) * D;
  const int nrows = min(kF8Bc, a.Nkv - kt * kF8Bc);
  for (int i = threadIdx.x; i < kF8Bc * D / 8; i += 256) {
    const int r = i / (D / 8), g = i % (D / 8);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < nrows) x = *(const u32x4*)(v + 8 * (size_t)i);
    *(u32x4*)(tile + r * (2 * D) + ((g ^ swz(r)) << 4)) = x;
  }
  __syncthreads();
  const float s = f8_qscale(a.amax[a.B * a.Hq + a.B * a.Hkv + head]);
  uint8_t* out = a.vt8 + ((size_t)head * a.nkt + kt) * D * kF8Bc;
  // each thread: columns 2 c2 and 2 c2 + 1 (one 4-byte read per key) at
  // positions p0 .. p0 + 15, i.e. 16 bytes of two rows of V8^T
  for (int i = threadIdx.x; i < D * 2; i += 256) {
    const int c2 = i >> 2, p0 = 16 * (i & 3);
    const int g = c2 >> 2, within = 4 * (c2 & 3);  // granule of the pair, its byte offset
    float f0[16], f1[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = f8_key_of_pos(p0 + e);
      const uint32_t w = *(const uint32_t*)(tile + r * (2 * D) + ((g ^ swz(r)) << 4) + within);
      f0[e] = E::to_f32((uint16_t)(w & 0xffff)) * s;
      f1[e] = E::to_f32((uint16_t)(w >> 16)) * s;
    }
    u32x4 w0, w1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      w0[c] = f8_pack4(f0[4 * c], f0[4 * c + 1], f0[4 * c + 2], f0[4 * c + 3]);
      w1[c] = f8_pack4(f1[4 * c], f1[4 * c + 1], f1[4 * c + 2], f1[4 * c + 3]);
    }
    *(u32x4*)(out + (size_t)(2 * c2) * kF8Bc + p0) = w0;
    *(u32x4*)(out + (size_t)(2 * c2 + 1) * kF8Bc + p0) = w1;
  }
}

// ---------------------------------------------------------------------------
// MFMA 32x32x64 with fp8 e4m3 A and B (cbsz = blgp = 0): C[32x32] += A[32x64]
// B[64x32]. Lane l holds row l % 32 of A and column l % 32 of B, 32 bytes
// each: lane half h the k positions 32 h .. 32 h + 31 of A's row and of B's
// column in one fixed order (any order serves, the same for A and B). A and B
// in VGPRs; C in AGPRs (C_AGPR) or VGPRs. Hazard padding as for the 16-bit
// MFMA: FIRST pads 4 wait states before (a VALU write of B just before),
// LAST pads 21 after (a VALU read of the result next).
// ---------------------------------------------------------------------------
#define FFPA_F8_ASM(CA, ZERO, PRE, POST)                                                                     \
  if constexpr (ZERO)                                                                                        \
    asm volatile(PRE "v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" POST : "=&" CA(acc) : "v"(a), "v"(b));      \
  else                                                                                                       \
    asm volatile(PRE "v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" POST : "+" CA(acc) : "v"(a), "v"(b));
template <bool C_AGPR, bool ZERO = false, bool FIRST = false, bool LAST = false>
__device__ inline void mfma_f8_asm(f32x16& acc, u32x8 a, u32x8 b) {
  if constexpr (C_AGPR) {
    if constexpr (FIRST && LAST) { FFPA_F8_ASM("a", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    else if constexpr (FIRST) { FFPA_F8_ASM("a", ZERO, "s_nop 4\n", "") }
    else if constexpr (LAST) { FFPA_F8_ASM("a", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    else { FFPA_F8_ASM("a", ZERO, "", "") }
  } else {
    if constexpr (FIRST && LAST) { FFPA_F8_ASM("v", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    else if constexpr (FIRST) { FFPA_F8_ASM("v", ZERO, "s_nop 4\n", "") }
    else if constexpr (LAST) { FFPA_F8_ASM("v", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    else { FFPA_F8_ASM("v", ZERO, "", "") }
  }
}
#undef FFPA_F8_ASM

// ---------------------------------------------------------------------------
// The attention kernel. Workgroup = 4 waves x 32 query rows of one head; per
// tile of 64 keys, double-buffered in LDS (K8 tile: 64 rows x D bytes, 16-byte
// granule g of row r at dense_pos(D / 16, r, g); V8^T tile: D rows x 64
// bytes, granule g of row d at g ^ ((d / 4) % 4)):
//   S^T (keys x queries, two blocks of 32 keys) = K8 Q8^T, A = K8 from LDS,
//   B = Q8 from registers (loaded once);
//   P = 2^(S - m) per query (a lane's query is lane % 32; its two lane halves
//   hold different keys), quantised to e4m3 (64 P) in registers: exactly the
//   B operand of O^T += V8^T P^T, whose A is the V8^T tile;
//   O^T (d x queries) in AGPRs: a lane holds its own query, so the online
//   softmax rescale is per lane.
// ---------------------------------------------------------------------------
template <int D>
constexpr int f8_lds_bytes() {
  return 2 * 2 * kF8Bc * D;
}

template <int D, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fwd_fp8_kernel(Fp8Args a) {
  static_assert(D % 64 == 0 && D >= 128 && D <= 512, "D must be a multiple of 64 in [128, 512]");
  using E = Elem<BF16>;
  constexpr int NST = D / 64;  // k-steps of S (64 d each)
  constexpr int NDB = D / 32;  // d-blocks of O
  constexpr int G = D / 16;    // 16-byte granules per K row
  constexpr int KT = kF8Bc * D;  // bytes of a K (or V^T) tile
  constexpr int NKC = D / 64;  // copy instructions per wave and tile, each tensor
  constexpr int kAhead = 4;    // K operand fragments read ahead of their MFMA
  constexpr int kAheadV = D == 512 ? 3 : 4;  // V^T fragments (registers are short at 512)

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5, l32 = lane & 31;

  const int t = xcd_logical(blockIdx.x, a.total_wg);
  int qt = t % a.n_qtiles;
  const int bh = t / a.n_qtiles;
  if (a.causal) qt = a.n_qtiles - 1 - qt;  // longest rows first
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int bhk = b * a.Hkv + hk;
  const int q0 = qt * kF8Rows, qw = q0 + 32 * wave, my_q = qw + l32;

  const float dq = f8_descale(a.amax[bh]);
  const float dk = f8_descale(a.amax[a.B * a.Hq + bhk]);
  const float dv = f8_descale(a.amax[a.B * a.Hq + a.B * a.Hkv + bhk]);
  const float sc = a.scale_log2 * dq * dk;  // log2-domain factor of the fp8 product

  // Q8 of the lane's query (rows past Nq read row Nq - 1, never stored):
  // step st, lane half h: bytes 64 st + 32 h .. + 31
  u32x8 qf[NST];
  {
    const uint8_t* qrow = a.q8 + ((size_t)bh * a.Nq + min(my_q, a.Nq - 1)) * D + 32 * hi;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const u32x4 x0 = *(const u32x4*)(qrow + 64 * st), x1 = *(const u32x4*)(qrow + 64 * st + 16);
      qf[st] = u32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
  }

  const uint32_t k_bytes = (uint32_t)a.Nkv * D;  // rows at or past Nkv read as zeros
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(a.k8 + (size_t)bhk * a.Nkv * D, k_bytes);
  const __amdgpu_buffer_rsrc_t Vr =
      make_rsrc(a.vt8 + (size_t)bhk * a.nkt * KT, (uint32_t)a.nkt * KT);
  // copy instruction n (n = wave + 4 r) fills 1 KiB of a tile: slots 64 n + lane
  uint32_t koff[NKC], voff[NKC];
#pragma unroll
  for (int r = 0; r < NKC; ++r) {
    const int s = 64 * (wave + 4 * r) + lane;
    const int kr = s / G, kg = dense_pos(G, kr, s % G);
    koff[r] = (uint32_t)(kr * D + 16 * kg);
    const int vd = s >> 2, vg = (s & 3) ^ ((vd >> 2) & 3);
    voff[r] = (uint32_t)(vd * kF8Bc + 16 * vg);
  }
  // K(j) and V^T(j) go to the buffer pair j % 2 (K at 0, V^T at KT)
  auto issue_k = [&](int j) {
    FFPA_LDS char* kb = smem + (j & 1) * 2 * KT;
#pragma unroll
    for (int r = 0; r < NKC; ++r) dma16(Kr, koff[r] + (uint32_t)j * KT, kb + (wave + 4 * r) * 1024);
  };
  auto issue_v = [&](int j) {
    FFPA_LDS char* vb = smem + (j & 1) * 2 * KT + KT;
#pragma unroll
    for (int r = 0; r < NKC; ++r) dma16(Vr, voff[r] + (uint32_t)j * KT, vb + (wave + 4 * r) * 1024);
  };

  int n_tiles = (a.Nkv + kF8Bc - 1) / kF8Bc;
  if (a.causal) n_tiles = min(n_tiles, (min(q0 + kF8Rows, a.Nq) + kF8Bc - 1) / kF8Bc);

  f32x16 o_acc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o_acc[d] = f32x16{};
  float m_ref = -INFINITY, l_run = 0.f;

  // LDS addresses of this lane's fragments, relative to a tile buffer
  uint32_t kaddr[2][NST];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int r = 32 * kb + l32, g = 4 * st + 2 * hi;
      kaddr[kb][st] = (uint32_t)(r * D + 16 * dense_pos(G, r, g));
    }
  // V^T row d = 32 db + l32 has the swizzle of l32 ((d / 4) % 4 = (l32 / 4) % 4):
  // one base, d-block db at + 32 x 64 db bytes
  const uint32_t vaddr0 = (uint32_t)(KT + l32 * kF8Bc + 16 * ((2 * hi) ^ ((l32 >> 2) & 3)));
  // the second granule of a fragment: logical g + 1 (g even), stored at
  // dense_pos(g + 1) = dense_pos(g) ^ 1 for both layouts (their swizzles flip
  // whole aligned pairs or leave bit 0 alone)
  auto frag = [&](const FFPA_LDS char* base, uint32_t off) {
    const u32x4 x0 = lds_read16(base + off), x1 = lds_read16(base + (off ^ 16u));
    return u32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };

  // The loop is pipelined over tiles: iteration j computes the scores
  // S(j + 1) on the matrix cores while the VALU turns the scores of tile j
  // into quantised P (exponentials at the MFMA slots), then the products
  // O^T += V8^T(j) P8^T(j) while the VALU scales and masks S(j + 1) and takes
  // its row max. K(j + 1) and V^T(j) must be in LDS at iteration j: the
  // copies of K(j + 2) and V^T(j + 1) are issued at its top, into the
  // buffers that K(j) and V^T(j - 1) have left.
  float tv[32];             // scaled, masked scores of the tile the VALU works on
  float mx = -INFINITY;     // their row max (lane half's keys, then both)
  // scores of tile jn from s_acc, element pair c (2c, 2c + 1), into tv / mx
  auto score_pair = [&](const f32x16* s_acc, int jn, bool edge, int c) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * c + e, kb = i >> 4, r = i & 15;
      float x = s_acc[kb][r] * sc;
      if (edge) {
        const int key = jn * kF8Bc + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool dead = (key >= a.Nkv) | (a.causal & (key > my_q));
        x = dead ? -INFINITY : x;
      }
      tv[i] = x;
      mx = fmaxf(mx, x);
    }
  };
  // only a tile that reaches past Nkv or past the wave's first query (causal)
  // has keys to mask; the test is uniform over the wave
  auto is_edge = [&](int jn) { return jn * kF8Bc + kF8Bc > a.Nkv || (a.causal && jn * kF8Bc + kF8Bc - 1 > qw); };
  // S^T(jn) = K8(jn) Q8^T, the two 32-key blocks interleaved; `slot(u)` runs
  // beside MFMA u (VALU work pinned there)
  auto s_chain = [&](f32x16* s_acc, int jn, auto&& slot) {
    const FFPA_LDS char* buf = smem + (jn & 1) * 2 * KT;
    u32x8 kf[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) kf[u] = frag(buf, kaddr[u & 1][u >> 1]);
#pragma unroll
    for (int u = 0; u < 2 * NST; ++u) {
      const u32x8 x = kf[u % kAhead];
      if (u + kAhead < 2 * NST) kf[u % kAhead] = frag(buf, kaddr[(u + kAhead) & 1][(u + kAhead) >> 1]);
      const int kb = u & 1, st = u >> 1;
      if (st == 0) mfma_f8_asm<false, true, true>(s_acc[kb], x, qf[st]);
      else if (u == 2 * NST - 1) mfma_f8_asm<false, false, false, true>(s_acc[kb], x, qf[st]);
      else mfma_f8_asm<false>(s_acc[kb], x, qf[st]);
      slot(u);
    }
    pin_after_pad(s_acc[0]);
    pin_after_pad(s_acc[1]);
  };

  f32x16 s_acc[2];
  if (n_tiles > 0) {
    issue_k(0);
    if (n_tiles > 1) issue_k(1);
    issue_v(0);
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    s_chain(s_acc, 0, [&](int) {});
#pragma unroll
    for (int c = 0; c < 16; ++c) score_pair(s_acc, 0, true, c);
    mx = fmaxf(mx, swap_halves(mx));
  }
  for (int j = 0; j < n_tiles; ++j) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) asm volatile("" : "+a"(o_acc[d]));
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();  // K(j + 1) and V^T(j) landed everywhere; K(j), V^T(j - 1) read by all
    if (j + 2 < n_tiles) issue_k(j + 2);
    if (j + 1 < n_tiles) issue_v(j + 1);

    // a row's reference max rises to the tile's max (O and l follow) when
    // that passes it by more than tau, and only then: P stays below 2^tau,
    // 64 P inside e4m3's range, and each row's reference depends on its own
    // scores alone (the ballot only skips the rescale when no row rises)
    const bool rise = mx > m_ref + kF8Tau;
    if (__builtin_amdgcn_ballot_w64(rise) != 0) {
      const float m_new = rise ? mx : m_ref;
      const float alpha = rise ? exp2_fast(m_ref - m_new) : 1.f;  // m_ref = -inf: 0, nothing held yet
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        scale_agpr16(o_acc[d], alpha);
        asm volatile("" : "+a"(o_acc[d]));
      }
    }
    // 64 P = 2^(t - (m - 6)): the P scale folded into the exponent; l_run
    // sums 64 P (the 64 is taken out at the end)
    static_assert(kF8PScale == 64.f && kF8PLog2 == 6.f, "P scale and its log2 go together");
    const float m_use = (m_ref == -INFINITY ? 0.f : m_ref) - kF8PLog2;
    float pv[32];
    u32x8 pf;
    // exponentials of element pair c (2c, 2c + 1), packed by fours
    auto exp_pair = [&](int c) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * c + e;
        asm volatile("" : "+v"(tv[i]));
        pv[i] = exp2_fast(tv[i] - m_use);
        l_run += pv[i];
      }
      if (c & 1) {
        const int w = c >> 1;
        pf[w] = f8_pack4(pv[4 * w], pv[4 * w + 1], pv[4 * w + 2], pv[4 * w + 3]);
        asm volatile("" : "+v"(pf[w]));
      }
    };
    // the 16 pairs spread over the 2 NST MFMA slots of the next scores
    auto exp_slot = [&](int u) {
#pragma unroll
      for (int c = 0; c < 16; ++c)
        if ((c * 2 * NST) / 16 == u) exp_pair(c);
    };
    // on the last tile the chain runs on a stale K buffer (no copy is in
    // flight into it) and its scores are never used: one spare chain per
    // workgroup instead of a branch in every slot
    s_chain(s_acc, j + 1, exp_slot);
    asm volatile("" : "+v"(pf));

    // O^T += V8^T(j) P8^T(j) over the d-blocks, beside the scores of S(j + 1)
    // (edge: it has keys to mask)
    auto pv_phase = [&](bool edge) {
      const FFPA_LDS char* buf = smem + (j & 1) * 2 * KT;
      u32x8 vf[kAheadV];
#pragma unroll
      for (int u = 0; u < kAheadV; ++u) vf[u] = frag(buf, vaddr0 + 32 * kF8Bc * u);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x8 x = vf[db % kAheadV];
        if (db + kAheadV < NDB) vf[db % kAheadV] = frag(buf, vaddr0 + 32 * kF8Bc * (db + kAheadV));
        if (db == 0) mfma_f8_asm<true, false, true>(o_acc[db], x, pf);
        else if (db == NDB - 1) mfma_f8_asm<true, false, false, true>(o_acc[db], x, pf);
        else mfma_f8_asm<true>(o_acc[db], x, pf);
        // 32 scores over the NDB slots (NDB = D / 32 >= 4)
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if ((c * NDB) / 16 == db) score_pair(s_acc, j + 1, edge, c);
      }
    };
    mx = -INFINITY;
    pv_phase(is_edge(j + 1));
    mx = fmaxf(mx, swap_halves(mx));
  }

  // epilogue: both lane halves hold partial row sums of the lane's query
  const float l_tot = l_run + swap_halves(l_run);  // 64 l
  const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * dv;
  if (my_q < a.Nq) {
    typename E::scalar* orow = (typename E::scalar*)a.o + ((size_t)bh * a.Nq + my_q) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      asm volatile("" : "+a"(o_acc[db]));
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16& x = o_acc[db];
        const uint32_t w0 = E::pack2(x[4 * g4] * inv, x[4 * g4 + 1] * inv);
        const uint32_t w1 = E::pack2(x[4 * g4 + 2] * inv, x[4 * g4 + 3] * inv);
        *(uint2*)(orow + 32 * db + 8 * g4 + 4 * hi) = make_uint2(w0, w1);
      }
    }
    if (a.lse != nullptr && hi == 0)
      a.lse[(size_t)bh * a.Nq + my_q] = l_tot > 0.f ? (m_ref + __log2f(l_tot) - kF8PLog2) * kLn2 : -INFINITY;
  }
}

// Bytes of the workspace: amax (3 x B Hq floats, padded), Q8, K8, V8^T.
__host__ __device__ inline size_t f8_amax_bytes(int B, int Hq) {
  return ((size_t)3 * B * Hq * 4 + 255) / 256 * 256;
}
__host__ __device__ inline size_t f8_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int D) {
  const size_t nkt = (size_t)(Nkv + kF8Bc - 1) / kF8Bc;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return f8_amax_bytes(B, Hq) + up((size_t)B * Hq * Nq * D) + up((size_t)B * Hkv * Nkv * D) +
         up((size_t)B * Hkv * nkt * D * kF8Bc);
}

// Host launcher: zero amax, amax pass, quantisation of Q, K and V^T, then the
// attention kernel. The caller has set every pointer of `a` (workspace
// carved as f8_workspace_bytes describes) and checked the grid sizes.
template <int D, bool BF16>
hipError_t launch_fwd_fp8(const Fp8Args& a, hipStream_t stream) {
  constexpr int lds = f8_lds_bytes<D>();
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_fp8_kernel<D, BF16>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)f8_quant_vt_kernel<D, BF16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kF8Bc * D * 2);
    return e;
  }();
  if (attr != hipSuccess) return attr;
  const int n_amax = a.B * a.Hq + 2 * a.B * a.Hkv;
  hipLaunchKernelGGL(f8_zero_kernel<D>, dim3((n_amax + 255) / 256), dim3(256), 0, stream, a.amax, n_amax);
  const int amax_wg = a.B * a.Hq * ((a.Nq + kF8AmaxRows - 1) / kF8AmaxRows) +
                      2 * a.B * a.Hkv * ((a.Nkv + kF8AmaxRows - 1) / kF8AmaxRows);
  hipLaunchKernelGGL((f8_amax_kernel<D, BF16>), dim3(amax_wg), dim3(256), 0, stream, a);
  const int64_t n16 = ((int64_t)a.B * a.Hq * a.Nq + (int64_t)a.B * a.Hkv * a.Nkv) * (D / 16);
  hipLaunchKernelGGL((f8_quant_qk_kernel<D, BF16>), dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((f8_quant_vt_kernel<D, BF16>), dim3(a.B * a.Hkv * a.nkt), dim3(256), kF8Bc * D * 2, stream, a);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, BF16>), dim3(a.total_wg), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
