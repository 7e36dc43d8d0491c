// Backward attention kernels (head dimensions that are multiples of 64, up to
// 1024): dQ, dK and dV of O = softmax(scale * Q K^T + mask) V, given dO and
// the forward's per-row logsumexp.
//
// The gradients are those of the "naive_math" definition (section 3 of the
// attention-kernel-profiler design document), in the standard flash form
// that the "FFPA Attention Benchmark" backward counts as 5 GEMMs:
//     P  = exp(scale S + mask - lse),  S = Q K^T        (recomputed, never stored)
//     dV = P^T dO,   dP = dO V^T,   delta_i = sum_d dO_id O_id
//     dS = P o (dP - delta),   dK = scale dS^T Q,   dQ = scale dS K
// with GQA gradients summed over the query heads of a group. Three launches:
//  1. bwd_prep_kernel: delta and lse * log2(e) per row into the workspace
//     (padded rows get delta = 0 and +inf, which makes their P zero);
//  2. bwd_dkdv_kernel: one workgroup per 64 keys of a (batch, kv head),
//     looping over every query tile of every query head of the group;
//  3. bwd_dq_kernel: one workgroup per 64 queries of a (batch, head),
//     looping over the key tiles.
//
// Register budget at D = 512. A workgroup is 4 waves = 2 row blocks of 32
// (keys for dK/dV, queries for dQ) x 2 halves of D. A wave holds the
// operands of its rows for its half of D (K and V, or Q and dO: 128 AGPRs)
// and the fp32 gradient accumulators of its rows for that half (256
// registers). Each score-like product (S and dP) is a contraction over all
// of D: a wave computes the partial sum over its half, the two waves of a
// row block swap partial sums through LDS, and both then hold the full S and
// dP tile (the sum a + b is the same in either order, so both see identical
// values). Every product is an MFMA 32x32x16 with one operand streamed from
// LDS: per wave and 32 x 32 tile, 4 products of D/2 = 64 MFMAs.
//
// Staged tiles (Q and dO, or K and V): 32 rows, double-buffered, copied
// straight from global memory into LDS. Every row takes 1 KiB: the two
// 512-byte halves hold the two halves of D, and granule g (8 elements) of a
// half is stored at g ^ swz4(row), which keeps both the 16-byte row reads
// and the transposed 8-byte reads conflict-free.
//
// Above D = 512 (BwdShape): the same waves split D in four parts instead of
// two (D is padded with zero columns to a multiple of 128, so a part is a
// whole number of 32-column blocks, at most 256), a workgroup covers one row
// block of 32, the partial sums are reduced over four waves, and the staged
// rows take 2 KiB (four 512-byte part slots). Two such tiles fill 128 KiB,
// so they are single-buffered: the next tile is copied once every wave is
// done with the current one.
#pragma once

#include "ffpa_common.hpp"
#include "fwd_vt.hpp"

namespace ffpa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B, Hq, Nq] natural log, from the forward
  void* dq;
  void* dk;
  void* dv;
  const void* mask;  // key bias [Nkv] or per-query mask [Nq, Nkv] in the input dtype, or null
  int mask_rows;     // 0, 1 or Nq
  float* delta;      // workspace [B * Hq * nq_pad]
  float* lse2;       // workspace [B * Hq * nq_pad]: lse * log2(e), +inf for dead and padded rows
  int B, Hq, Hkv, Nq, Nkv;
  int nq_pad;        // Nq rounded up to 64
  int causal;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  int wg_dkdv;       // B * Hkv * ceil(Nkv / 64)
  int wg_dq;         // B * Hq * ceil(Nq / 64)
  // stored-dS path (null ds: dQ recomputes S and dP instead)
  void* ds;          // workspace: dS in blocks of 32 queries x 32 keys (bwd_ds_block)
  void* kt;          // workspace: K^T in blocks of 32 keys (fwd_vt.hpp layout)
  int nqt, nkt;      // ceil(Nq / 32), ceil(Nkv / 32)
  int nkv_pad;       // Nkv rounded up to 64
  int wg_dq_ds;      // B * Hq * ceil(Nq / bwd_dq_ds_rows(D))
  DropParams drop;   // dropout of the forward (drop.t = 0: none)
  int bh0;           // flattened query head of head 0 of this launch (the dropout counter)
};

// The stored dS. Block (bh, qt, kt) holds dS[q][key] for the 32 queries of
// tile qt and the 32 keys of tile kt of head bh = b Hq + h: 2 KiB, 32 rows of
// 64 bytes (one per query), whose positions hold the keys in the order
// vt_key(pos) of fwd_vt.hpp, so that 16-byte granule 2 t2 + h of a row
// pairs with granule 2 t2 + h of a K^T row of the same tile (the MFMA
// operand pieces of key step t2 and lane half h).
__host__ __device__ inline size_t bwd_ds_block(int bh, int qt, int kt, int nqt, int nkt) {
  return (((size_t)bh * nqt + qt) * nkt + kt) * 2048;
}
// queries per workgroup of the stored-dS dQ kernel
__host__ __device__ inline int bwd_dq_ds_rows(int D) { return D > 512 ? 64 : 128; }

constexpr int kBwdRows = 32;                       // rows per staged tile
constexpr int kBwdPartBytes = 512;                 // LDS slot of one part of a row
constexpr int kBwdXchg = 8 * 1024;                 // per wave: partial S and dP tiles, fp32
constexpr int kBwdLds = 160 * 1024;                // tiles (128 KiB) + swap area (32 KiB)
constexpr int kBwdPad = 64;                        // workspace row padding

// This lane's index in the wave (0..63), computed where it is used: the asm
// is opaque, so the compiler keeps no lane-id register live across a loop
// (which it would for threadIdx.x) when registers are short.
__device__ inline int lane_id_here() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n v_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

// A compile-time integer as a type, to instantiate a generic lambda per value.
template <int I>
struct IntTag {
  static constexpr int value = I;
};

// Zero that the compiler cannot see through: an MFMA operand register that
// holds zero padding then stays a register (a visible constant would be
// rematerialised by VALU writes right before each MFMA, inside its hazard
// window).
__device__ inline u32x4 opaque_zero4() {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return u32x4{z, z, z, z};
}

// How a head dimension is split over the 4 waves of a workgroup.
template <int D>
struct BwdShape {
  static constexpr int NP = D > 512 ? 4 : 2;                        // parts of D
  static constexpr int DP = NP == 2 ? D : (D + 127) / 128 * 128;    // D padded with zero columns
  static constexpr int DW = DP / NP;                                // columns per part
  static constexpr int ROWB = NP * kBwdPartBytes;                   // LDS bytes per staged row
  static constexpr int TILE = kBwdRows * ROWB;                      // bytes per staged tile
  static constexpr int NB = NP == 2 ? 2 : 1;                        // buffers per staged tensor
  static constexpr int RB = 4 / NP;                                 // row blocks of 32 per workgroup
  static constexpr int ROWS = kBwdRows * RB;                        // keys (dK/dV) or queries (dQ) per workgroup
  static_assert(DW % 32 == 0 && DW <= 256, "a part is whole 32-column blocks, at most 256");
  static_assert(4 * NB * TILE / 2 + 4 * kBwdXchg <= kBwdLds, "LDS budget");
};
// rows per workgroup of the two main kernels (host side: grid sizes)
inline int bwd_rows_per_wg(int D) { return D > 512 ? kBwdRows : 2 * kBwdRows; }

// ---------------------------------------------------------------------------
// Shared pieces of the two main kernels.
// ---------------------------------------------------------------------------

// Copy rows row0 .. row0 + 31 of a [rows, D] tensor (buffer resource `rs`)
// into a staged tile at `dst`. Wave w issues rows w, w + 4, ...; lane t of a
// row writes slot t % 32 of half t / 32, which holds the logical granule
// (t % 32) ^ swz4(row) of that half. The whole offset sits in the range-
// checked per-lane offset: rows past the end and granules past D/2 read as
// zeros (the latter without memory traffic).
// Copy instruction n fills 1 KiB: row n / S, part slots 2 (n % S) and
// 2 (n % S) + 1 (S = ROWB / 1 KiB); lane t writes slot t % 32 of part
// 2 (n % S) + t / 32. Columns at or past D (zero padding) are never loaded.
template <int D>
__device__ inline void bwd_copy_row(__amdgpu_buffer_rsrc_t rs, FFPA_LDS char* dst, int row0,
                                    int wave, int lane, int r) {
  using S = BwdShape<D>;
  constexpr int SUB = S::ROWB / 1024;
  const int u = lane & 31;
  const int n = wave + 4 * r;
  const int row = n / SUB, part = 2 * (n % SUB) + (lane >> 5);
  const int gl = u ^ swz4(row);
  const int col = part * S::DW + 8 * gl;
  const bool ok = gl < S::DW / 8 && (S::DP == D || col < D);
  const uint32_t lanepart = ok ? (uint32_t)col << 1 : 0x80000000u;
  dma16(rs, lanepart + (uint32_t)(row0 + row) * (D * 2), dst + n * 1024);
}
template <int D>
__device__ inline void bwd_copy_tile(__amdgpu_buffer_rsrc_t rs, FFPA_LDS char* dst, int row0,
                                     int wave, int lane) {
#pragma unroll
  for (int r = 0; r < kBwdRows * BwdShape<D>::ROWB / 1024 / 4; ++r) bwd_copy_row<D>(rs, dst, row0, wave, lane, r);
}

// The 16 copies of a wave for the next pair of tiles (8 rows of each),
// spread over the first `span` steps of a phase: copy c goes at step c span / 16.
template <int D>
__device__ inline void bwd_copy_spread(__amdgpu_buffer_rsrc_t ra, FFPA_LDS char* da,
                                       __amdgpu_buffer_rsrc_t rb, FFPA_LDS char* db, int row0,
                                       int wave, int lane, int st, int span) {
#pragma unroll
  for (int c = 0; c < 2 * kBwdRows / 4; ++c)
    if ((c * span) / (2 * kBwdRows / 4) == st) {
      if (c & 1) bwd_copy_row<D>(rb, db, row0, wave, lane, c >> 1);
      else bwd_copy_row<D>(ra, da, row0, wave, lane, c >> 1);
    }
}

// 16-byte row reads (MFMA A operand, m = row): lane l reads row l % 32,
// granule 2 st + l / 32 of part `hf`, st = 8 a + c. Per-lane bases for c.
template <int ROWB>
__device__ inline void bwd_row_bases(int ln, int hf, uint32_t* ax) {
  const int r = ln & 31, h = ln >> 5, x = swz4(r);
#pragma unroll
  for (int c = 0; c < 8; ++c)
    ax[c] = (uint32_t)(r * ROWB + hf * kBwdPartBytes + (((2 * c + h) ^ x) << 4));
}
__device__ inline uint32_t bwd_row_addr(const uint32_t* ax, int st) { return ax[st & 7] + 256 * (st >> 3); }

// Transposed reads (MFMA A operand, m = column d, k = row): for d-block db
// of half `hf` and row group t2, lane l gets column 32 db + l % 32 of rows
// 16 t2 + 8 (e / 4) + 4 (l / 32) + e % 4, e = 0..7 (two ds_read_b64_tr_b16).
// That row order matches the C layout of a 32x32 MFMA result whose m index
// is the row, so a P or dS tile feeds the B operand straight from registers.
template <int ROWB>
__device__ inline void bwd_tr_bases(int ln, int hf, uint32_t* tx) {
  const int G = ln >> 4, gi = ln & 15;
  const int vrow = 4 * (G >> 1) + (gi >> 2);
  const int y = 2 * (G & 1) + ((gi & 3) >> 1);
#pragma unroll
  for (int r8 = 0; r8 < 2; ++r8) {
    const int row = vrow + 8 * r8, x = swz4(row);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      tx[4 * r8 + e] = (uint32_t)(row * ROWB + hf * kBwdPartBytes + (((4 * e + y) ^ x) << 4) +
                                  (gi & 1) * 8);
  }
}
template <int ROWB>
__device__ inline u32x4 bwd_tr_read(const FFPA_LDS char* tile, const uint32_t* tx, int db, int t2) {
  const uint32_t off = 256 * (db >> 2) + 16 * t2 * ROWB;
  return join8(lds_read_tr(tile + tx[db & 3] + off), lds_read_tr(tile + tx[4 + (db & 3)] + off));
}

// Swap partial products with the waves holding the other parts of D for the
// same rows and add them up: afterwards s and p hold the full contractions.
// Every wave of a row block forms the same sum in the same order (part 0
// first), so all of them hold identical values. Contains a workgroup barrier
// (every wave calls it).
template <int NP>
__device__ inline void bwd_exchange(FFPA_LDS char* xbase, int wave, int lane, f32x16& s, f32x16& p) {
  FFPA_LDS f32x4* mine = (FFPA_LDS f32x4*)(xbase + wave * kBwdXchg) + lane;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mine[64 * j] = f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
    mine[64 * (4 + j)] = f32x4{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
  }
  wait_lgkm0();
  barrier();
  if constexpr (NP == 2) {
    // a + b is the same in either order
    const FFPA_LDS f32x4* other = (const FFPA_LDS f32x4*)(xbase + (wave ^ 1) * kBwdXchg) + lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 x = other[64 * j], y = other[64 * (4 + j)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[4 * j + e] += x[e];
        p[4 * j + e] += y[e];
      }
    }
  } else {
    // every part read back from LDS, the own one included, and summed in
    // place in part order
    const int first = wave - wave % NP;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const FFPA_LDS f32x4* src = (const FFPA_LDS f32x4*)(xbase + (first + q) * kBwdXchg) + lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 x = src[64 * j], y = src[64 * (4 + j)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[4 * j + e] = q == 0 ? x[e] : s[4 * j + e] + x[e];
          p[4 * j + e] = q == 0 ? y[e] : p[4 * j + e] + y[e];
        }
      }
    }
  }
}

// Partial products S (or S^T) and dP (or dP^T) over one half of D: A
// fragments are rows of the staged tiles `ta` and `tb`, B fragments the
// register operands `fa` and `fb` (AGPRs). The chains end padded for the
// VALU/LDS reads of their results.
template <bool BF16, int NS, int AHEAD = 3, class StepFn>
__device__ inline void bwd_partials(const FFPA_LDS char* ta, const FFPA_LDS char* tb, const uint32_t* ax,
                                    const u32x4* fa, const u32x4* fb, f32x16& s, f32x16& p,
                                    StepFn&& at_step) {
  constexpr int kAhead = NS < AHEAD ? NS : AHEAD;  // LDS reads in flight
  u32x4 xa[kAhead], xb[kAhead];
#pragma unroll
  for (int st = 0; st < kAhead; ++st) {
    xa[st] = lds_read16(ta + bwd_row_addr(ax, st));
    xb[st] = lds_read16(tb + bwd_row_addr(ax, st));
  }
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    at_step(st);
    const u32x4 x = xa[st % kAhead], y = xb[st % kAhead];
    if (st + kAhead < NS) {
      xa[st % kAhead] = lds_read16(ta + bwd_row_addr(ax, st + kAhead));
      xb[st % kAhead] = lds_read16(tb + bwd_row_addr(ax, st + kAhead));
    }
    if (st == 0) {
      mfma32_asm<BF16, true, false, true>(s, x, fa[st]);
      mfma32_asm<BF16, true, false, true>(p, y, fb[st]);
    } else if (st == NS - 1) {
      mfma32_asm<BF16, true, false>(s, x, fa[st]);
      mfma32_asm<BF16, true, false, false, false, true>(p, y, fb[st]);
      pin_after_pad(s);
    } else {
      mfma32_asm<BF16, true, false>(s, x, fa[st]);
      mfma32_asm<BF16, true, false>(p, y, fb[st]);
    }
  }
}

// Rows r = lane % 32 of a [32, D/2] fp32 result held transposed in MFMA
// accumulators (acc[db][4 g4 + e] = element (r, 32 db + 8 g4 + 4 (lane/32) + e)),
// scaled by `mul`, converted and written to a 512-byte-pitch LDS staging area
// (granule g of row r at g ^ (r % 16)).
template <bool BF16, int NDB>
__device__ inline void bwd_stage_rows(FFPA_LDS char* st, const f32x16* acc, float mul, int lane) {
  const int r = lane & 31, hie = lane >> 5;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const u32x2 w = {Elem<BF16>::pack2(acc[db][4 * g4] * mul, acc[db][4 * g4 + 1] * mul),
                       Elem<BF16>::pack2(acc[db][4 * g4 + 2] * mul, acc[db][4 * g4 + 3] * mul)};
      const int g = 4 * db + g4;
      *(FFPA_LDS u32x2*)(st + r * 512 + ((g ^ (r & 15)) << 4) + 8 * hie) = w;
    }
}

// Store `rows` (<= 32) staged rows of part `hf` to dst (row pitch D
// elements, dst at the part's first column), 16 bytes per lane and
// instruction; columns at or past D (zero padding) are not stored.
template <int D, class T>
__device__ inline void bwd_store_rows(T* dst, const FFPA_LDS char* st, int rows, int hf, int lane) {
  using S = BwdShape<D>;
  constexpr int SG = S::DW / 8;  // granules per staged row
  const int gmax = S::DP == D ? SG : min(SG, (D - hf * S::DW) / 8);
#pragma unroll
  for (int it = 0; it < SG / 2; ++it) {
    const int c = it * 64 + lane;
    const int r = c / SG, g = c % SG;
    const u32x4 x = *(const FFPA_LDS u32x4*)(st + r * 512 + ((g ^ (r & 15)) << 4));
    if (r < rows && g < gmax) *(u32x4*)(dst + (size_t)r * D + 8 * g) = x;
  }
}

// ---------------------------------------------------------------------------
// 1. delta_i = sum_d dO_id O_id and lse_i * log2(e), one wave per row.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  using T = typename Elem<BF16>::scalar;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.Hq * a.nq_pad) return;
  const int64_t bh = row / a.nq_pad;
  const int qi = (int)(row % a.nq_pad);
  float dsum = 0.f, l2 = INFINITY;
  if (qi < a.Nq) {
    const size_t base = ((size_t)bh * a.Nq + qi) * D;
    const T* O = (const T*)a.o + base;
    const T* dO = (const T*)a.dout + base;
    float acc = 0.f;
    for (int gi = lane; gi < D / 8; gi += 64) {
      const u32x4 x = *(const u32x4*)(O + 8 * gi), y = *(const u32x4*)(dO + 8 * gi);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += Elem<BF16>::to_f32((uint16_t)(x[e] & 0xffff)) * Elem<BF16>::to_f32((uint16_t)(y[e] & 0xffff));
        acc += Elem<BF16>::to_f32((uint16_t)(x[e] >> 16)) * Elem<BF16>::to_f32((uint16_t)(y[e] >> 16));
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    dsum = acc;
    const float l = a.lse[(size_t)bh * a.Nq + qi];
    l2 = l == -INFINITY ? INFINITY : l * kLog2e;  // a dead row has P = 0
  }
  if (lane == 0) {
    a.delta[row] = dsum;
    a.lse2[row] = l2;
  }
}

// ---------------------------------------------------------------------------
// 2. dK and dV. Wave (kb, hf) owns keys kw = 64 kt + 32 kb .. +31 and half hf
// of D. Per query tile (32 rows of one query head):
//    S, dP (32 q x 32 keys) partial over the half, swapped, summed;
//    P = 2^(scale_log2 S + bias_log2 - lse2), dS = P (dP - delta);
//    dV^T[half] += dO^T P,  dK^T[half] += Q^T dS.
// Accumulators: dV^T in AGPRs, dK^T in VGPRs (m = d, n = key).
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool ROWMASK, bool DROP = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdArgs a) {
  static_assert(D % 64 == 0 && D <= 1024, "D must be a multiple of 64, at most 1024");
  using E = Elem<BF16>;
  using T = typename E::scalar;
  using V8 = typename E::vec8;
  using Sh = BwdShape<D>;
  constexpr int DW = Sh::DW, NS = DW / 16, NDB = DW / 32;
  constexpr int QB = 0, OB = Sh::NB * Sh::TILE, XB = 2 * Sh::NB * Sh::TILE;
  constexpr int NT = 2 * NDB;                   // phase-2 steps per accumulator set
  constexpr int kTAhead = NT < 4 ? NT : 4;      // transposed-read lookahead
  // single buffer (D > 512): from 192 columns per part the dV^T and dK^T
  // products run one after the other so that the next dO tile is copied
  // during the latter (D = 1024: 5.6 % faster; 576: 1.3 % slower)
  constexpr bool kSplit = Sh::NB == 1 && DW >= 192;

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb = wave / Sh::NP, hf = wave % Sh::NP;

  const int n_kt = (a.Nkv + Sh::ROWS - 1) / Sh::ROWS;
  int kt, bhk;
  if (a.causal) {
    // the work of a key block falls with its index: blocks go out in that
    // order over all heads at once, longest first, so that list scheduling
    // evens out the triangle whatever the number of heads (XCD ranges of
    // one head's blocks would give some XCDs only long blocks)
    const int nh = a.wg_dkdv / n_kt;
    kt = blockIdx.x / nh;
    bhk = blockIdx.x % nh;
  } else {
    const int t = xcd_logical(blockIdx.x, a.wg_dkdv);
    kt = t % n_kt;
    bhk = t / n_kt;
  }
  const int hk = bhk % a.Hkv, b = bhk / a.Hkv;
  const int g = a.Hq / a.Hkv;
  const int kw = kt * Sh::ROWS + 32 * kb;

  // K and V of the wave's keys, its part of D: B operands (k = d, n = key);
  // padding columns (at or past D) are zeros
  u32x4 kf[NS], vf[NS];
  {
    const int key = min(kw + (lane & 31), a.Nkv - 1);  // keys past the end: never stored
    const int col0 = hf * DW + 8 * (lane >> 5);
    const size_t off = ((size_t)(b * a.Hkv + hk) * a.Nkv + key) * D + col0;
    const u32x4* kp = (const u32x4*)((const T*)a.k + off);
    const u32x4* vp = (const u32x4*)((const T*)a.v + off);
    const u32x4 z = opaque_zero4();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bool in = Sh::DP == D || col0 + 16 * st < D;
      kf[st] = in ? kp[2 * st] : z;
      vf[st] = in ? vp[2 * st] : z;
    }
    if constexpr (Sh::DP != D) {
      // settle the operands in AGPRs once (not copied in before every MFMA)
#pragma unroll
      for (int st = 0; st < NS; ++st) asm volatile("" : "+a"(kf[st]), "+a"(vf[st]));
    }
  }
  wait_vmcnt0_visible();
  float bias2 = 0.f;  // this lane's key bias, log2 domain
  // per-query mask: a separate instance, so the common one keeps its registers
  constexpr bool row_mask = ROWMASK;
  // lse2 and delta of the next tile are loaded during this one, except in the
  // per-query-mask instance, which needs those registers
  constexpr bool kPrefetch = !ROWMASK;
  if (a.mask != nullptr && !row_mask) {
    const int key = kw + (lane & 31);
    bias2 = key < a.Nkv ? E::to_f32(((const uint16_t*)a.mask)[key]) * kLog2e : -INFINITY;
  }

  const int n_qt = (a.Nq + kBwdRows - 1) / kBwdRows;
  const int qt0 = a.causal ? min(kt * Sh::ROWS / kBwdRows, n_qt) : 0;  // earlier query tiles see none of these keys
  const int per_head = n_qt - qt0;
  const int n_it = g * per_head;
  const uint32_t q_bytes = (uint32_t)a.Nq * D * 2;

  auto issue = [&](int it) {
    const int hh = hk * g + it / per_head;
    const int qt = qt0 + it % per_head;
    const size_t hoff = (size_t)(b * a.Hq + hh) * a.Nq * D * 2;
    const int s = it % Sh::NB;
    const int ln = lane_id_here();
    bwd_copy_tile<D>(make_rsrc((const char*)a.q + hoff, q_bytes), smem + QB + s * Sh::TILE, qt * kBwdRows, wave, ln);
    bwd_copy_tile<D>(make_rsrc((const char*)a.dout + hoff, q_bytes), smem + OB + s * Sh::TILE, qt * kBwdRows, wave, ln);
  };
  // single buffer: the tile of one tensor (Q if `of_q`, else dO) of iteration `it`
  auto issue_one = [&](int it, bool of_q) {
    const int hh = hk * g + it / per_head;
    const int qt = qt0 + it % per_head;
    const size_t hoff = (size_t)(b * a.Hq + hh) * a.Nq * D * 2;
    const int ln = lane_id_here();
    bwd_copy_tile<D>(make_rsrc((const char*)(of_q ? a.q : a.dout) + hoff, q_bytes), smem + (of_q ? QB : OB),
                     qt * kBwdRows, wave, ln);
  };

  f32x16 dv[NDB], dk[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dv[i] = f32x16{};
    dk[i] = f32x16{};
  }
  // lse2 and delta of iteration `it`, rows 8 j + 4 hi + 0..3 of its tile
  f32x4 l2n[4], dln[4];
  auto load_rows = [&](int it) {
    const int hh = hk * g + it / per_head;
    const int qt = qt0 + it % per_head;
    const size_t rb = (size_t)(b * a.Hq + hh) * a.nq_pad + qt * kBwdRows + 4 * (lane_id_here() >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      l2n[j] = *(const f32x4*)(a.lse2 + rb + 8 * j);
      dln[j] = *(const f32x4*)(a.delta + rb + 8 * j);
    }
  };
  if (n_it > 0) {
    if constexpr (kPrefetch) load_rows(0);
    issue(0);
  }

  for (int it = 0; it < n_it; ++it) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      asm volatile("" : "+a"(dv[d]));
      asm volatile("" : "+v"(dk[d]));
    }
    const int hh = hk * g + it / per_head;
    const int qt = qt0 + it % per_head;
    const int s = it % Sh::NB;
    const FFPA_LDS char* qtile = smem + QB + s * Sh::TILE;
    const FFPA_LDS char* otile = smem + OB + s * Sh::TILE;
    const int lj = lane_id_here();
    const int hij = lj >> 5;
    const int my_k = kw + (lj & 31);

    wait_vmcnt<0>();  // this wave's copies of tile `it` landed ...
    wait_lgkm0();
    barrier();        // ... everyone's; tile it - 1 and the swap area are free

    // lse2 and delta of rows 8 j + 4 hi + 0..3 of the tile: loaded during
    // the previous tile (see load_rows), complete since the wait above; the
    // empty asm makes the compiler's own wait for them fall here, before
    // this tile's copies are issued (a wait after them would hold for them).
    // (The per-query-mask instance has no registers to spare for the
    // prefetch: it loads them here.)
    if constexpr (!kPrefetch) load_rows(it);
    f32x4 l2[4], dl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      l2[j] = l2n[j];
      dl[j] = dln[j];
      if constexpr (kPrefetch) asm volatile("" ::"v"(l2[j]), "v"(dl[j]));
    }
    // dropout keep bit i: the lane's key against query 8 (i / 4) + i % 4 + 4 hi
    // of the tile (made before the products, while fewer registers are live)
    const uint32_t keep =
        DROP ? drop_bits_col(a.drop, a.bh0 + b * a.Hq + hh, my_k, qt * kBwdRows + 4 * hij) : 0u;
    // S = Q K^T and dP = dO V^T (32 q x 32 keys), partial over this half of
    // D; the copies of the next tile go out during its first half
    f32x16 sacc, pacc;
    {
      const bool has_next = it + 1 < n_it;
      const int hn = hk * g + (it + 1) / per_head;
      const int qn = qt0 + (it + 1) % per_head;
      const size_t hoff = (size_t)(b * a.Hq + hn) * a.Nq * D * 2;
      const __amdgpu_buffer_rsrc_t Qn = make_rsrc((const char*)a.q + hoff, q_bytes);
      const __amdgpu_buffer_rsrc_t On = make_rsrc((const char*)a.dout + hoff, q_bytes);
      FFPA_LDS char* qd = smem + QB + (s ^ 1) * Sh::TILE;
      FFPA_LDS char* od = smem + OB + (s ^ 1) * Sh::TILE;
      const int lc = lane_id_here();
      uint32_t ax[8];
      bwd_row_bases<Sh::ROWB>(lj, hf, ax);
      bwd_partials<BF16, NS>(qtile, otile, ax, kf, vf, sacc, pacc, [&](int st) {
        // double-buffered: the next tile's copies go out here
        if (Sh::NB == 2 && has_next)
          bwd_copy_spread<D>(Qn, qd, On, od, qn * kBwdRows, wave, lc, st, NS > 1 ? NS / 2 : 1);
      });
    }
    bwd_exchange<Sh::NP>(smem + XB, wave, lj, sacc, pacc);

    // P and dS; register i holds query 8 (i / 4) + 4 hi + i % 4 of the tile
    float pv[16], dsv[16];
    const int qg0 = qt * kBwdRows + 4 * hij;
    // the causal test is a separate instance of the loop (uniform branch),
    // so that non-causal tiles run no compares
    // dropout (Z, scale c): P o Z c feeds dV (c applied at the end) and
    // dS = P o (dP o Z c - delta)
    auto p_ds = [&](auto causal_tag) {
      constexpr bool CAUSAL = decltype(causal_tag)::value;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = i >> 2, e = i & 3;
        float x;
        if constexpr (row_mask) {
          // per-query mask: entry (row, my_k), rows clamped to the last one
          const int qr = min(qg0 + 8 * j + e, a.Nq - 1);
          const float bv = E::to_f32(((const uint16_t*)a.mask)[(size_t)qr * a.Nkv + min(my_k, a.Nkv - 1)]);
          const float bias_i = my_k < a.Nkv ? bv * kLog2e : -INFINITY;
          x = fmaf(sacc[i], a.scale_log2, bias_i) - l2[j][e];
        } else {
          x = fmaf(sacc[i], a.scale_log2, bias2 - l2[j][e]);
        }
        if constexpr (CAUSAL) x = my_k > qg0 + 8 * j + e ? -INFINITY : x;
        const float p = exp2_fast(x);
        if constexpr (DROP) {
          // the scale of the kept P is applied to dV at the end
          pv[i] = keep_if_bit(p, keep, i);
          dsv[i] = p * (keep_if_bit(pacc[i] * a.drop.scale, keep, i) - dl[j][e]);
        } else {
          pv[i] = p;
          dsv[i] = p * (pacc[i] - dl[j][e]);
        }
      }
    };
    if (a.causal && kw + 31 > qt * kBwdRows) p_ds(BoolTag<true>{});
    else p_ds(BoolTag<false>{});
    V8 pf[2], sf[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const float* x = &pv[8 * t2];
      const float* y = &dsv[8 * t2];
      pf[t2] = pack8<BF16>(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
      sf[t2] = pack8<BF16>(y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7]);
    }
    // every VALU write of the MFMA B operands happens before this point; the
    // first MFMA below pads for the last of them
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(pf[t2]), "+v"(sf[t2]));

    // dS for the dQ pass: lane (key, h) holds dS of 16 queries of its key;
    // the dQ product needs each query's keys in one lane. One MFMA per wave
    // transposes a half: with A = the packed dS of query step t2 = hf (m =
    // key, k = 16 queries) and B = the 0/1 matrix that maps k back to its
    // query n, C[key][q] = dS[q][key] for the 16 queries of the step (exact:
    // each sum has one nonzero term). Lane (q, h) of C then holds keys
    // 8 (i / 4) + 4 h + i % 4, i.e. positions 8 h .. 8 h + 7 and 16 + 8 h ..
    // of the block row in vt_key order: two 16-byte stores.
    // (t2 a constant in each instance: an operand picked by a runtime index
    // made the compiler rebuild the packed tiles inside the products below)
    auto store_ds = [&](auto t2_tag, const V8& sfa) {
      constexpr int t2 = decltype(t2_tag)::value;
      const int qn = lj & 31, hn = lj >> 5;
      const int r = qn - 16 * t2;  // the query's index within the step
      const bool mine = (unsigned)r < 16u;
      // the 1 sits at element e = 4 ((r / 8) % 2) + r % 4 of lane half (r / 4) % 2
      const int e = 4 * ((r >> 3) & 1) + (r & 3);
      const uint32_t one = (mine && ((r >> 2) & 1) == hn) ? (BF16 ? 0x3F80u : 0x3C00u) << (16 * (e & 1)) : 0u;
      u32x4 ib;
#pragma unroll
      for (int w = 0; w < 4; ++w) ib[w] = (e >> 1) == w ? one : 0u;
      f32x16 tr;
      mfma32_asm<BF16, false, false, true, true, true>(tr, __builtin_bit_cast(u32x4, sfa), ib);
      // the values are 16-bit numbers held exactly in fp32: bf16 keeps the
      // high halves (one byte permute per pair), fp16 converts exactly
      auto pk = [&](float x, float y) -> uint32_t {
        if constexpr (BF16)
          return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, y), __builtin_bit_cast(uint32_t, x), 0x07060302u);
        else
          return E::pack2(x, y);
      };
      if (mine) {
        char* blk = (char*)a.ds + bwd_ds_block(b * a.Hq + hh, qt, kw / 32, a.nqt, a.nkt) + qn * 64;
        const u32x4 g0 = {pk(tr[0], tr[1]), pk(tr[2], tr[3]), pk(tr[4], tr[5]), pk(tr[6], tr[7])};
        const u32x4 g1 = {pk(tr[8], tr[9]), pk(tr[10], tr[11]), pk(tr[12], tr[13]), pk(tr[14], tr[15])};
        // non-temporal: dS is read once, by the dQ pass; kept out of the
        // way of the Q and dO tiles in L2 (8 % faster than plain stores)
        __builtin_nontemporal_store(g0, (u32x4*)(blk + 16 * hn));
        __builtin_nontemporal_store(g1, (u32x4*)(blk + 16 * (2 + hn)));
      }
      // the stores go out here, not among the products below (their data
      // would stay live there)
      asm volatile("" ::: "memory");
    };
    // (causal: a block above the diagonal, all zero and never read, is not stored)
    if (a.ds != nullptr && kw < a.Nkv && !(a.causal && kw / 32 > qt)) {
      if (hf == 0) store_ds(IntTag<0>{}, sf[0]);
      else if (hf == 1) store_ds(IntTag<1>{}, sf[1]);
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(pf[t2]), "+v"(sf[t2]));

    // the next tile's lse2 and delta, waited for at its barrier
    if constexpr (kPrefetch) {
      if (it + 1 < n_it) load_rows(it + 1);
    }

    // dV^T += dO^T P and dK^T += Q^T dS over the half's d-blocks; step
    // st = NDB t2 + db, so consecutive MFMAs use different accumulators
    {
      uint32_t tx[8];
      {
        const int lv = lane_id_here();
        bwd_tr_bases<Sh::ROWB>(lv, hf, tx);
      }
      if constexpr (!kSplit) {
        u32x4 fo[kTAhead], fq[kTAhead];
#pragma unroll
        for (int st = 0; st < kTAhead; ++st) {
          fo[st] = bwd_tr_read<Sh::ROWB>(otile, tx, st % NDB, st / NDB);
          fq[st] = bwd_tr_read<Sh::ROWB>(qtile, tx, st % NDB, st / NDB);
        }
#pragma unroll
        for (int st = 0; st < NT; ++st) {
          const int db = st % NDB, t2 = st / NDB;
          const u32x4 x = fo[st % kTAhead], y = fq[st % kTAhead];
          if (st + kTAhead < NT) {
            fo[st % kTAhead] = bwd_tr_read<Sh::ROWB>(otile, tx, (st + kTAhead) % NDB, (st + kTAhead) / NDB);
            fq[st % kTAhead] = bwd_tr_read<Sh::ROWB>(qtile, tx, (st + kTAhead) % NDB, (st + kTAhead) / NDB);
          }
          const u32x4 pb = __builtin_bit_cast(u32x4, pf[t2]), sb = __builtin_bit_cast(u32x4, sf[t2]);
          if (st == 0) mfma32_asm<BF16, false, true, false, true>(dv[db], x, pb);
          else mfma32_asm<BF16, false, true>(dv[db], x, pb);
          // the iteration's last MFMA pads: the compiler may copy accumulators
          // on the loop's exit or back edge right after it
          if (st == NT - 1) mfma32_asm<BF16, false, false, false, false, true>(dk[db], y, sb);
          else mfma32_asm<BF16, false, false>(dk[db], y, sb);
        }
      } else {
        // all of dV^T first; once every wave is done with the dO tile, the
        // next one is copied during the dK^T products, and the next Q tile
        // after them (each chain pads at both ends: other code sits between)
        u32x4 fr[kTAhead];
#pragma unroll
        for (int st = 0; st < kTAhead; ++st) fr[st] = bwd_tr_read<Sh::ROWB>(otile, tx, st % NDB, st / NDB);
#pragma unroll
        for (int st = 0; st < NT; ++st) {
          const int db = st % NDB, t2 = st / NDB;
          const u32x4 x = fr[st % kTAhead];
          if (st + kTAhead < NT) fr[st % kTAhead] = bwd_tr_read<Sh::ROWB>(otile, tx, (st + kTAhead) % NDB, (st + kTAhead) / NDB);
          const u32x4 pb = __builtin_bit_cast(u32x4, pf[t2]);
          if (st == 0) mfma32_asm<BF16, false, true, false, true>(dv[db], x, pb);
          else if (st == NT - 1) mfma32_asm<BF16, false, true, false, false, true>(dv[db], x, pb);
          else mfma32_asm<BF16, false, true>(dv[db], x, pb);
        }
        if (it + 1 < n_it) {
          wait_lgkm0();
          barrier();
          issue_one(it + 1, false);
        }
#pragma unroll
        for (int st = 0; st < kTAhead; ++st) fr[st] = bwd_tr_read<Sh::ROWB>(qtile, tx, st % NDB, st / NDB);
#pragma unroll
        for (int st = 0; st < NT; ++st) {
          const int db = st % NDB, t2 = st / NDB;
          const u32x4 y = fr[st % kTAhead];
          if (st + kTAhead < NT) fr[st % kTAhead] = bwd_tr_read<Sh::ROWB>(qtile, tx, (st + kTAhead) % NDB, (st + kTAhead) / NDB);
          const u32x4 sb = __builtin_bit_cast(u32x4, sf[t2]);
          if (st == 0) mfma32_asm<BF16, false, false, false, true>(dk[db], y, sb);
          else if (st == NT - 1) mfma32_asm<BF16, false, false, false, false, true>(dk[db], y, sb);
          else mfma32_asm<BF16, false, false>(dk[db], y, sb);
        }
        if (it + 1 < n_it) {
          wait_lgkm0();
          barrier();
          issue_one(it + 1, true);
        }
      }
    }
    if constexpr (Sh::NB == 1 && !kSplit) {
      // single buffer: the next tile is copied once every wave is done with this one
      if (it + 1 < n_it) {
        wait_lgkm0();
        barrier();
        issue(it + 1);
      }
    }
  }
  wait_vmcnt<0>();
  // the accumulators were last written by MFMAs issued as inline asm: pad
  // before the epilogue reads them
  asm volatile("s_nop 7\n s_nop 7\n s_nop 4" ::: "memory");
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    asm volatile("" : "+a"(dv[d]));
    asm volatile("" : "+v"(dk[d]));
  }

  // ---- epilogue: each wave stages its 32 keys x D/2 of dV and dK (16 KiB
  // each) in LDS, then stores them as contiguous 16-byte pieces
  wait_lgkm0();
  barrier();
  FFPA_LDS char* stg = smem + wave * 2 * 16384;
  const int le = lane_id_here();
  bwd_stage_rows<BF16, NDB>(stg, dv, DROP ? a.drop.scale : 1.f, le);
  bwd_stage_rows<BF16, NDB>(stg + 16384, dk, a.scale, le);
  {
    const size_t row0 = ((size_t)(b * a.Hkv + hk) * a.Nkv + kw) * D + hf * DW;
    const int rows = min(kBwdRows, a.Nkv - kw);
    bwd_store_rows<D>((T*)a.dv + row0, stg, rows, hf, le);
    bwd_store_rows<D>((T*)a.dk + row0, stg + 16384, rows, hf, le);
  }
}

// ---------------------------------------------------------------------------
// 3. dQ. Wave (qb, hf) owns queries qw = 64 qblk + 32 qb .. +31 and half hf
// of D. Per key tile (32 keys):
//    S^T, dP^T (32 keys x 32 q) partial over the half, swapped, summed;
//    P = 2^(scale_log2 S + bias_log2 - lse2), dS = P (dP - delta);
//    dQ^T[half] += K^T dS^T   (accumulators in AGPRs, m = d, n = query).
// ---------------------------------------------------------------------------
template <int D, bool BF16, bool DROP = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(BwdArgs a) {
  static_assert(D % 64 == 0 && D <= 1024, "D must be a multiple of 64, at most 1024");
  using E = Elem<BF16>;
  using T = typename E::scalar;
  using V8 = typename E::vec8;
  using Sh = BwdShape<D>;
  constexpr int DW = Sh::DW, NS = DW / 16, NDB = DW / 32;
  constexpr int KB = 0, VB = Sh::NB * Sh::TILE, XB = 2 * Sh::NB * Sh::TILE;
  constexpr int NT = 2 * NDB;
  constexpr int kTAhead = NT < 6 ? NT : 6;

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qb = wave / Sh::NP, hf = wave % Sh::NP;

  const int n_qb = (a.Nq + Sh::ROWS - 1) / Sh::ROWS;
  int qblk, bh;
  if (a.causal) {
    // longest rows (last query blocks) first over all heads at once, as in
    // the dK/dV pass
    const int nh = a.wg_dq / n_qb;
    qblk = n_qb - 1 - (int)blockIdx.x / nh;
    bh = blockIdx.x % nh;
  } else {
    const int t = xcd_logical(blockIdx.x, a.wg_dq);
    qblk = t % n_qb;
    bh = t / n_qb;
  }
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int qw = qblk * Sh::ROWS + 32 * qb;

  // Q and dO of the wave's rows, its part of D: B operands (k = d, n =
  // query); padding columns (at or past D) are zeros
  u32x4 qf[NS], of[NS];
  {
    const int qr = min(qw + (lane & 31), a.Nq - 1);  // rows past the end: never stored
    const int col0 = hf * DW + 8 * (lane >> 5);
    const size_t off = ((size_t)(b * a.Hq + h) * a.Nq + qr) * D + col0;
    const u32x4* qp = (const u32x4*)((const T*)a.q + off);
    const u32x4* op = (const u32x4*)((const T*)a.dout + off);
    const u32x4 z = opaque_zero4();
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bool in = Sh::DP == D || col0 + 16 * st < D;
      qf[st] = in ? qp[2 * st] : z;
      of[st] = in ? op[2 * st] : z;
    }
    if constexpr (Sh::DP != D) {
      // settle the operands in AGPRs once (not copied in before every MFMA)
#pragma unroll
      for (int st = 0; st < NS; ++st) asm volatile("" : "+a"(qf[st]), "+a"(of[st]));
    }
  }
  // this lane's row: lse2 (+inf past Nq) and delta, from the padded workspace
  const size_t wrow = (size_t)(b * a.Hq + h) * a.nq_pad + qw + (lane & 31);
  const float lse2_me = a.lse2[wrow];
  const float dl_me = a.delta[wrow];
  wait_vmcnt0_visible();

  int kv_end = a.Nkv;
  if (a.causal) kv_end = min(kv_end, min(qblk * Sh::ROWS + Sh::ROWS, a.Nq));  // keys <= last row of the block
  const int n_kt = (kv_end + kBwdRows - 1) / kBwdRows;
  const size_t kvoff = (size_t)(b * a.Hkv + hk) * a.Nkv * D * 2;
  const uint32_t kv_bytes = (uint32_t)a.Nkv * D * 2;
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc((const char*)a.k + kvoff, kv_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc((const char*)a.v + kvoff, kv_bytes);
  const uint16_t* mk = (const uint16_t*)a.mask;

  auto issue = [&](int j) {
    const int s = j % Sh::NB;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    bwd_copy_tile<D>(Kr, smem + KB + s * Sh::TILE, j * kBwdRows, wave, ln);
    bwd_copy_tile<D>(Vr, smem + VB + s * Sh::TILE, j * kBwdRows, wave, ln);
  };

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};
  // mask entries of key tile jt for this lane's keys (register i: key
  // 32 jt + 4 hi + 8 (i / 4) + i % 4): key bias, or row my_q of a per-query
  // mask (clamped to the last row). Loaded one tile ahead, during the
  // previous tile's dQ products, so that the wait for them comes before the
  // tile's copies are in flight.
  float bn[16];
  auto load_bias = [&](int jt) {
    const int kgb = jt * kBwdRows + 4 * (lane >> 5);
    const uint16_t* mrow = mk + (a.mask_rows > 1 ? (size_t)min(qw + (lane & 31), a.Nq - 1) * a.Nkv : 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) bn[i] = E::to_f32(mrow[min(kgb + 8 * (i >> 2) + (i & 3), a.Nkv - 1)]);
  };
  if (n_kt > 0) {
    if (mk != nullptr) load_bias(0);
    issue(0);
  }

  for (int j = 0; j < n_kt; ++j) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) asm volatile("" : "+a"(dq[d]));
    const int s = j % Sh::NB;
    const FFPA_LDS char* ktile = smem + KB + s * Sh::TILE;
    const FFPA_LDS char* vtile = smem + VB + s * Sh::TILE;
    int lj = lane;
    asm volatile("" : "+v"(lj));
    const int hij = lj >> 5;
    const int my_q = qw + (lj & 31);
    const int kg0 = j * kBwdRows + 4 * hij;  // register i holds key kg0 + 8 (i / 4) + i % 4

    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();

    float bias2[16];
    if (mk != nullptr) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kg0 + 8 * (i >> 2) + (i & 3);
        float bv = bn[i];
        asm volatile("" : "+v"(bv));  // the compiler's wait for the load falls here
        bias2[i] = key < a.Nkv ? bv * kLog2e : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) bias2[i] = kg0 + 8 * (i >> 2) + (i & 3) < a.Nkv ? 0.f : -INFINITY;
    }
    // dropout keep bit i for the lane's row against key kg0 + 8 (i / 4) +
    // i % 4 (made before the products, while fewer registers are live)
    const uint32_t keep = DROP ? drop_bits_row(a.drop, a.bh0 + bh, my_q, kg0) : 0u;
    // S^T = K Q^T and dP^T = V dO^T (32 keys x 32 q), partial over the
    // half; the copies of the next tile go out during its first half
    f32x16 sacc, pacc;
    {
      const bool has_next = j + 1 < n_kt;
      FFPA_LDS char* kd = smem + KB + (s ^ 1) * Sh::TILE;
      FFPA_LDS char* vd = smem + VB + (s ^ 1) * Sh::TILE;
      int lc = lane;
      asm volatile("" : "+v"(lc));
      uint32_t ax[8];
      bwd_row_bases<Sh::ROWB>(lj, hf, ax);
      bwd_partials<BF16, NS>(ktile, vtile, ax, qf, of, sacc, pacc, [&](int st) {
        // double-buffered: the next tile's copies go out here
        if (Sh::NB == 2 && has_next)
          bwd_copy_spread<D>(Kr, kd, Vr, vd, (j + 1) * kBwdRows, wave, lc, st, NS > 1 ? NS / 2 : 1);
      });
    }
    bwd_exchange<Sh::NP>(smem + XB, wave, lj, sacc, pacc);

    float dsv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = fmaf(sacc[i], a.scale_log2, bias2[i]) - lse2_me;
      if (a.causal && kg0 + 8 * (i >> 2) + (i & 3) > my_q) x = -INFINITY;
      const float p = exp2_fast(x);
      if constexpr (DROP) {
        dsv[i] = p * (keep_if_bit(pacc[i] * a.drop.scale, keep, i) - dl_me);
      } else {
        dsv[i] = p * (pacc[i] - dl_me);
      }
    }
    V8 sf[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const float* y = &dsv[8 * t2];
      sf[t2] = pack8<BF16>(y[0], y[1], y[2], y[3], y[4], y[5], y[6], y[7]);
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(sf[t2]));

    if (mk != nullptr && j + 1 < n_kt) load_bias(j + 1);

    // dQ^T += K^T dS^T over the half's d-blocks
    {
      uint32_t tx[8];
      {
        int lv = lane;
        asm volatile("" : "+v"(lv));
        bwd_tr_bases<Sh::ROWB>(lv, hf, tx);
      }
      u32x4 fk[kTAhead];
#pragma unroll
      for (int st = 0; st < kTAhead; ++st) fk[st] = bwd_tr_read<Sh::ROWB>(ktile, tx, st % NDB, st / NDB);
#pragma unroll
      for (int st = 0; st < NT; ++st) {
        const int db = st % NDB, t2 = st / NDB;
        const u32x4 x = fk[st % kTAhead];
        if (st + kTAhead < NT) fk[st % kTAhead] = bwd_tr_read<Sh::ROWB>(ktile, tx, (st + kTAhead) % NDB, (st + kTAhead) / NDB);
        const u32x4 sb = __builtin_bit_cast(u32x4, sf[t2]);
        // first MFMA pads for the VALU writes of dS; the last for accumulator
        // copies the compiler may place on the loop's exit or back edge
        if (st == 0 && NT == 1) mfma32_asm<BF16, false, true, false, true, true>(dq[db], x, sb);
        else if (st == 0) mfma32_asm<BF16, false, true, false, true>(dq[db], x, sb);
        else if (st == NT - 1) mfma32_asm<BF16, false, true, false, false, true>(dq[db], x, sb);
        else mfma32_asm<BF16, false, true>(dq[db], x, sb);
      }
    }
    if constexpr (Sh::NB == 1) {
      // single buffer: the next tile is copied once every wave is done with this one
      if (j + 1 < n_kt) {
        wait_lgkm0();
        barrier();
        issue(j + 1);
      }
    }
  }
  wait_vmcnt<0>();
  asm volatile("s_nop 7\n s_nop 7\n s_nop 4" ::: "memory");
#pragma unroll
  for (int d = 0; d < NDB; ++d) asm volatile("" : "+a"(dq[d]));

  wait_lgkm0();
  barrier();
  FFPA_LDS char* stg = smem + wave * 16384;
  bwd_stage_rows<BF16, NDB>(stg, dq, a.scale, lane);
  {
    const size_t row0 = ((size_t)(b * a.Hq + h) * a.Nq + qw) * D + hf * DW;
    bwd_store_rows<D>((T*)a.dq + row0, stg, min(kBwdRows, a.Nq - qw), hf, lane);
  }
}

// ---------------------------------------------------------------------------
// 3b. dQ from the stored dS: dQ^T += K^T dS^T per key tile, nothing
// recomputed. Wave (qb, hf) owns queries qw = ROWS qblk + 32 qb .. +31 and
// part hf of D (D <= 512: all of D, 4 query blocks per workgroup; above: two
// halves, 2 query blocks). The K^T tile (D rows of 32 keys, 64 bytes each,
// from the blocked transposed copy) is staged in LDS, double-buffered, and
// read with plain 16-byte reads as the A operand; the dS block of the wave's
// queries comes straight from global memory as the B operand, one tile
// ahead. Under causal masking the blocks above the diagonal were never
// written (their dS is zero): a wave skips the products of those tiles.
// ---------------------------------------------------------------------------
constexpr int kBwdDqDsLds = 128 * 1024;

template <int D, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dq_ds_kernel(BwdArgs a) {
  static_assert(D % 64 == 0 && D <= 1024, "D must be a multiple of 64, at most 1024");
  using E = Elem<BF16>;
  using T = typename E::scalar;
  constexpr int NQP = D > 512 ? 2 : 1;  // parts of D
  constexpr int DQ = D / NQP;           // columns per wave
  constexpr int NDB = DQ / 32;
  constexpr int ROWS = 32 * (4 / NQP);  // queries per workgroup
  constexpr int TILE = D * 64;          // bytes of a staged K^T tile
  constexpr int NVC = D / 64;           // copy instructions per wave and tile
  constexpr int NT = 2 * NDB;           // MFMA steps per tile: st = NDB t2 + db
  constexpr int kAhead = NT < 8 ? NT : 8;
  // accumulator blocks in AGPRs; the rest in VGPRs (all 256 AGPRs taken
  // makes the allocator spill)
  constexpr int kAcc = NDB < 12 ? NDB : 12;
  static_assert(2 * TILE <= kBwdDqDsLds && 4 * 32 * 1024 <= kBwdDqDsLds, "LDS budget");

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qb = wave / NQP, hf = wave % NQP;

  const int n_qb = (a.Nq + ROWS - 1) / ROWS;
  int qblk, bh;
  if (a.causal) {
    // longest rows (last query blocks) first over all heads at once, as in
    // the dK/dV pass
    const int nh = a.wg_dq_ds / n_qb;
    qblk = n_qb - 1 - (int)blockIdx.x / nh;
    bh = blockIdx.x % nh;
  } else {
    const int t = xcd_logical(blockIdx.x, a.wg_dq_ds);
    qblk = t % n_qb;
    bh = t / n_qb;
  }
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int qw = qblk * ROWS + 32 * qb;
  const int qt = qw / 32;

  int kv_end = a.Nkv;
  if (a.causal) kv_end = min(kv_end, min(qblk * ROWS + ROWS, a.Nq));  // keys <= last row of the block
  const int n_kt = (kv_end + 31) / 32;
  // tiles with products for this wave: all, or (causal) those with keys <= its last row
  int my_end = a.causal ? min(n_kt, qt + 1) : n_kt;
  if (qw >= a.Nq) my_end = 0;  // a block past the last query: no dS rows

  const uint32_t kt_bytes = (uint32_t)D * a.nkv_pad * 2;
  const __amdgpu_buffer_rsrc_t Ktr =
      make_rsrc((const char*)a.kt + (size_t)(b * a.Hkv + hk) * kt_bytes, kt_bytes);
  // this lane's dS pieces: row l % 32 of the wave's block, granule 2 t2 + l / 32
  const char* dsrow = (const char*)a.ds + (my_end > 0 ? bwd_ds_block(bh, qt, 0, a.nqt, a.nkt) : 0) +
                      (lane & 31) * 64 + (lane >> 5) * 16;

  // copy instruction n (n = wave + 4 r, r < NVC) fills LDS rows 16 n .. 16 n +
  // 15 of a tile: lane i writes slot i % 4 of row 16 n + i / 4, which holds
  // the logical granule (i % 4) ^ ((row / 4) % 4), and (row / 4) % 4 =
  // (i / 16) % 4 whatever n is
  uint32_t lo;
  {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    lo = (uint32_t)(ln >> 2) * 64 + (uint32_t)(((ln & 3) ^ ((ln >> 4) & 3)) << 4);
    asm volatile("" : "+v"(lo));
  }
  auto kt_copy = [&](int j, int r) {
    const int n = wave + 4 * r;
    dma16(Ktr, lo + (uint32_t)(16 * n) * 64 + (uint32_t)j * TILE, smem + (j & 1) * TILE + n * 1024);
  };

  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};
  u32x4 bn[2];  // dS pieces of the next tile
  auto load_ds = [&](int j) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      bn[t2] = __builtin_nontemporal_load((const u32x4*)(dsrow + (size_t)j * 2048 + 32 * t2));
  };
  if (n_kt > 0) {
    if (my_end > 0) load_ds(0);
    wait_vmcnt0_visible();
#pragma unroll
    for (int r = 0; r < NVC; ++r) kt_copy(0, r);
  }

  for (int j = 0; j < n_kt; ++j) {
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      if (d < kAcc) asm volatile("" : "+a"(dq[d]));
      else asm volatile("" : "+v"(dq[d]));
    }
    wait_vmcnt<0>();  // this wave's copies of tile j landed ...
    wait_lgkm0();
    barrier();        // ... everyone's; tile j - 1's buffer is free
    const bool more = j + 1 < n_kt;
    if (j < my_end) {
      u32x4 bc[2] = {bn[0], bn[1]};
      // the compiler's wait for the dS loads falls here, before any copy is in flight
      asm volatile("" ::"v"(bc[0]), "v"(bc[1]));
      if (j + 1 < my_end) load_ds(j + 1);
      uint32_t vx[2];
      {
        int lv = lane;
        asm volatile("" : "+v"(lv));
        const int r = lv & 31, hh = lv >> 5;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          vx[t2] = (uint32_t)((j & 1) * TILE + (DQ * hf + r) * 64 + (((2 * t2 + hh) ^ ((r >> 2) & 3)) << 4));
      }
      auto aread = [&](int st) { return lds_read16(smem + vx[st / NDB] + 2048 * (st % NDB)); };
      u32x4 af[kAhead];
#pragma unroll
      for (int st = 0; st < kAhead; ++st) af[st] = aread(st);
#pragma unroll
      for (int st = 0; st < NT; ++st) {
        // the next tile's copies, spread over the first half of the steps
#pragma unroll
        for (int r = 0; r < NVC; ++r)
          if (more && (r * (NT / 2)) / NVC == st) kt_copy(j + 1, r);
        const int db = st % NDB, t2 = st / NDB;
        const u32x4 x = af[st % kAhead];
        if (st + kAhead < NT) af[st % kAhead] = aread(st + kAhead);
        // the first MFMA pads for a VALU copy of the dS pieces, the last for
        // accumulator copies on the loop's exit or back edge
        if (db < kAcc) {
          if (st == 0) mfma32_asm<BF16, false, true, false, true>(dq[db], x, bc[t2]);
          else if (st == NT - 1) mfma32_asm<BF16, false, true, false, false, true>(dq[db], x, bc[t2]);
          else mfma32_asm<BF16, false, true>(dq[db], x, bc[t2]);
        } else {
          if (st == 0) mfma32_asm<BF16, false, false, false, true>(dq[db], x, bc[t2]);
          else if (st == NT - 1) mfma32_asm<BF16, false, false, false, false, true>(dq[db], x, bc[t2]);
          else mfma32_asm<BF16, false, false>(dq[db], x, bc[t2]);
        }
      }
    } else if (more) {
#pragma unroll
      for (int r = 0; r < NVC; ++r) kt_copy(j + 1, r);
    }
  }
  wait_vmcnt<0>();
  asm volatile("s_nop 7\n s_nop 7\n s_nop 4" ::: "memory");
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    if (d < kAcc) asm volatile("" : "+a"(dq[d]));
    else asm volatile("" : "+v"(dq[d]));
  }

  // ---- epilogue: 32 rows of the wave's part through LDS (1 KiB pitch,
  // granule g of row r at g ^ (r % 16)), then 16-byte stores along rows
  wait_lgkm0();
  barrier();
  FFPA_LDS char* stg = smem + wave * 32 * 1024;
  {
    const int r = lane & 31, hie = lane >> 5;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 w = {E::pack2(dq[db][4 * g4] * a.scale, dq[db][4 * g4 + 1] * a.scale),
                         E::pack2(dq[db][4 * g4 + 2] * a.scale, dq[db][4 * g4 + 3] * a.scale)};
        const int g = 4 * db + g4;
        *(FFPA_LDS u32x2*)(stg + r * 1024 + ((g ^ (r & 15)) << 4) + 8 * hie) = w;
      }
  }
  {
    constexpr int SG = DQ / 8;
    constexpr int NIT = (32 * SG + 63) / 64;
    T* dst = (T*)a.dq + ((size_t)bh * a.Nq + qw) * D + DQ * hf;
    const int rows = min(32, a.Nq - qw);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = it * 64 + lane;
      const int r = c / SG, g = c % SG;
      if (r < rows) {
        const u32x4 x = *(const FFPA_LDS u32x4*)(stg + r * 1024 + ((g ^ (r & 15)) << 4));
        *(u32x4*)(dst + (size_t)r * D + 8 * g) = x;
      }
    }
  }
}

// Sets the dynamic-LDS limit of every kernel launch_bwd<D, BF16> may enqueue.
// Called (through launch_bwd) before the first launch, so that a failure here
// leaves nothing enqueued.
template <int D, bool BF16>
hipError_t prepare_bwd() {
  static const hipError_t e = [] {
    const void* big[] = {(const void*)bwd_dkdv_kernel<D, BF16, false>, (const void*)bwd_dkdv_kernel<D, BF16, true>,
                         (const void*)bwd_dkdv_kernel<D, BF16, false, true>,
                         (const void*)bwd_dkdv_kernel<D, BF16, true, true>, (const void*)bwd_dq_kernel<D, BF16>,
                         (const void*)bwd_dq_kernel<D, BF16, true>};
    for (const void* k : big) {
      const hipError_t r = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kBwdLds);
      if (r != hipSuccess) return r;
    }
    return hipFuncSetAttribute((const void*)bwd_dq_ds_kernel<D, BF16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kBwdDqDsLds);
  }();
  return e;
}

// The arguments of a chunk of n kv heads starting at flattened kv head f0
// (f = b Hkv + hk): every tensor is [B, H, ...] contiguous, so heads f0 ..
// f0 + n - 1 (and their query heads f g .. f g + g - 1) are one contiguous
// run, and the chunk is the problem B = 1, Hkv = n, Hq = n g on offset
// pointers. The dS buffer is not offset: each chunk reuses it from the start.
template <int D>
BwdArgs bwd_chunk_args(const BwdArgs& a, int f0, int n) {
  const int g = a.Hq / a.Hkv;
  const size_t fq = (size_t)f0 * g;
  BwdArgs c = a;
  c.q = (const char*)a.q + fq * a.Nq * D * 2;
  c.o = (const char*)a.o + fq * a.Nq * D * 2;
  c.dout = (const char*)a.dout + fq * a.Nq * D * 2;
  c.dq = (char*)a.dq + fq * a.Nq * D * 2;
  c.lse = a.lse + fq * a.Nq;
  c.delta = a.delta + fq * a.nq_pad;
  c.lse2 = a.lse2 + fq * a.nq_pad;
  c.k = (const char*)a.k + (size_t)f0 * a.Nkv * D * 2;
  c.v = (const char*)a.v + (size_t)f0 * a.Nkv * D * 2;
  c.dk = (char*)a.dk + (size_t)f0 * a.Nkv * D * 2;
  c.dv = (char*)a.dv + (size_t)f0 * a.Nkv * D * 2;
  c.kt = (char*)a.kt + (size_t)f0 * D * a.nkv_pad * 2;
  c.B = 1;
  c.Hkv = n;
  c.Hq = n * g;
  c.bh0 = a.bh0 + (int)fq;
  const int rows = bwd_rows_per_wg(D), rq = bwd_dq_ds_rows(D);
  c.wg_dkdv = n * ((a.Nkv + rows - 1) / rows);
  c.wg_dq = n * g * ((a.Nq + rows - 1) / rows);
  c.wg_dq_ds = n * g * ((a.Nq + rq - 1) / rq);
  return c;
}

// Host launcher: the kernels in order on `stream`. With the stored-dS path
// (a.ds set) the dK/dV and dQ passes run per chunk of `chunk_kv` kv heads
// (the dS buffer holds one chunk); otherwise once over the whole problem.
// The caller has checked the grid sizes.
template <int D, bool BF16>
hipError_t launch_bwd(const BwdArgs& a, int chunk_kv, hipStream_t stream) {
  const hipError_t pe = prepare_bwd<D, BF16>();
  if (pe != hipSuccess) return pe;
  const bool rowmask = a.mask != nullptr && a.mask_rows > 1;
  const bool drop = a.drop.t != 0;
  auto kdkdv = drop ? (rowmask ? bwd_dkdv_kernel<D, BF16, true, true> : bwd_dkdv_kernel<D, BF16, false, true>)
                    : (rowmask ? bwd_dkdv_kernel<D, BF16, true> : bwd_dkdv_kernel<D, BF16, false>);
  auto kdq = drop ? bwd_dq_kernel<D, BF16, true> : bwd_dq_kernel<D, BF16>;
  const int64_t rows = (int64_t)a.B * a.Hq * a.nq_pad;
  hipLaunchKernelGGL((bwd_prep_kernel<D, BF16>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
  if (a.ds != nullptr) {
    // stored-dS path: K^T for the dQ pass, then per chunk dK/dV (which writes
    // the chunk's dS) and dQ = scale dS K
    const hipError_t e = launch_fwd_vt(a.k, a.kt, a.B * a.Hkv, a.Nkv, D, 32, stream);
    if (e != hipSuccess) return e;
    const int nkv = a.B * a.Hkv;
    for (int f0 = 0; f0 < nkv; f0 += chunk_kv) {
      const BwdArgs c = bwd_chunk_args<D>(a, f0, min(chunk_kv, nkv - f0));
      hipLaunchKernelGGL(kdkdv, dim3(c.wg_dkdv), dim3(256), kBwdLds, stream, c);
      hipLaunchKernelGGL((bwd_dq_ds_kernel<D, BF16>), dim3(c.wg_dq_ds), dim3(256), kBwdDqDsLds, stream, c);
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL(kdkdv, dim3(a.wg_dkdv), dim3(256), kBwdLds, stream, a);
  hipLaunchKernelGGL(kdq, dim3(a.wg_dq), dim3(256), kBwdLds, stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
