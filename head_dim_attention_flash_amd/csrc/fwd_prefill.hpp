// Forward attention kernel, 32 query rows per wave (head dimensions that are
// multiples of 64, up to 512; and 576 and 640 with the fp16 output
// accumulator and V staged from its transposed copy).
//
// What it computes: O = softmax(scale * Q K^T + mask) V and lse per row, the
// "naive_math" definition of section 3 of the attention-kernel-profiler design
// document, with the additive mask and GQA conventions of "FFPA Attention
// Benchmark" ("Quick Start") and the profiler's "gqa_4kv" entry. The scores
// are never materialised in memory: keys are visited in tiles of 64 and the
// softmax is carried online (running max and sum, output rescaled).
//
// Work decomposition (MI355X): one workgroup = 4 waves = 128 query rows of
// one (batch, head). Wave w owns 32 rows. Every wave computes
//     S^T (64 keys x 32 queries) = K_tile Q^T       (MFMA 32x32x16, A = K from LDS)
//     O^T (D x 32 queries)     += V_tile^T P^T      (MFMA 32x32x16, A = V^T from LDS)
// so that each lane's accumulators all belong to one query row (l % 32): the
// online-softmax rescale is a per-lane scalar and P goes from the S
// accumulators into the B operand of the second MFMA without leaving
// registers. With VT, V is staged from its transposed copy (fwd_vt.hpp), so
// both operands read from LDS are plain 16-byte reads; without it (problems
// with few queries per key, where the copy would not pay) V is staged like K
// and its fragments come from transposed 8-byte reads.
//
// Staging: one LDS buffer holds the K tile (64 keys x D, dense rows of D x 2
// bytes), another the V^T tile (D rows x 64 keys, 128 bytes per row) or the V
// tile (like K), all swizzled. The copy of V(j) is spread over the K(j) phase
// and the copy of K(j+1) over the V(j) phase, so each copy has one phase of
// MFMA work to land, and a tile costs two workgroup barriers. Copies go
// straight from global memory to LDS (buffer_load ... lds); the K and V
// buffer resources' ranges end at row Nkv, so rows past the end read as
// zeros, and V^T is zero past Nkv by construction.
#pragma once

#include "ffpa_common.hpp"
#include "fwd_vt.hpp"

namespace ffpa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* vt;     // V transposed (fwd_vt.hpp): [B, Hkv, D, nkv_pad] for the prefill
                      // kernel, [B, Hkv, nkv_pad / 32, D, 32] for the wide one
  int nkv_pad;        // Nkv rounded up to a multiple of 64
  void* o;
  float* lse;         // may be null
  const void* mask;   // may be null
  int B, Hq, Hkv, Nq, Nkv;
  int mask_rows;      // 0 (none), 1 (key bias) or Nq (per-query mask)
  int mask_stride;    // elements between mask rows read from global memory: 0 (key bias) or Nkv
  int bias_lds;       // 1: the key bias is staged in LDS after the tiles
  int causal;
  float scale_log2;   // scale * log2(e)
  int n_qtiles;
  int total_wg;
  DropParams drop;    // dropout (drop.t = 0: none)
};

constexpr int kFwdWaves = 4;
constexpr int kFwdRows = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBc = 64;                // keys per tile

// Every staged row takes 1 KiB of LDS whatever D is (up to 512): one copy
// instruction fills one row, the swizzle groups are all complete, and two
// 64-row tiles still fit. Above 512 (576, 640) a row takes D x 2 bytes: the
// two tiles then fill 144 or 160 KiB, and the epilogue stages each row in
// whole groups of 16 granules.
constexpr int kFwdRowBytes = 1024;
template <int D>
constexpr int fwd_row_bytes() {
  return D * 2 > kFwdRowBytes ? D * 2 : kFwdRowBytes;
}
template <int D>
constexpr int fwd_epi_pitch() {
  return D * 2 > kFwdRowBytes ? (D / 8 + 15) / 16 * 256 : kFwdRowBytes;
}

// LDS bytes of the K and V tile buffers.
template <int D>
constexpr int fwd_ring_bytes() {
  return 2 * kFwdBc * fwd_row_bytes<D>();
}
// LDS bytes of the epilogue's staging (the 32 rows of each of the 4 waves)
template <int D>
constexpr int fwd_epi_bytes() {
  return kFwdWaves * 32 * fwd_epi_pitch<D>();
}
// LDS bytes of the staged key bias (zero-padded to whole tiles).
__host__ __device__ inline int fwd_bias_bytes(int nkv) { return ((nkv + kFwdBc - 1) / kFwdBc) * kFwdBc * 2; }
// LDS bytes after the buffers and the bias: four restart flags.
constexpr int kFwdFlagBytes = 16;

// Online softmax without rescaling the fp32 output accumulators.
// Each row keeps a reference max m_ref (log2 domain) and accumulates
// P = 2^(t - m_ref). m_ref is set from the first tile in which the row sees an
// unmasked key. As long as every later score stays below m_ref + tau, P stays
// within 2^tau (representable in the MFMA operand type) and no accumulator
// ever needs a rescale. A tile that breaks the bound makes the whole
// workgroup restart its key loop with O and l zeroed and the raised m_ref;
// every restart lifts a row's reference by more than tau, so there are at most
// (range of the scores) / tau of them (none on typical data). The fp16
// accumulator path instead renormalises every tile (its scale is a VGPR op).
template <bool BF16>
constexpr float fwd_tau() {
  return BF16 ? 60.0f : 15.0f;  // P <= 2^15 < 65504 (fp16); bf16 has fp32's range
}
constexpr float kRescaleTau = 8.0f;  // fp16-accumulator path: move m_ref past this

template <int D, bool BF16, bool ACC16, bool VT, bool DROP = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fwd_prefill_kernel(FwdArgs a) {
  // above 512 the fp32 O no longer fits beside Q, and only the transposed V
  // layout (128-byte rows) keeps the V tile within the LDS
  static_assert(D % 64 == 0 && (D <= 512 || ((D == 576 || D == 640) && ACC16 && VT)),
                "D must be a multiple of 64, at most 512 (576, 640: fp16 accumulator, V^T staged)");
  static_assert(!(ACC16 && DROP), "dropout is built with fp32 accumulation");
  using E = Elem<BF16>;
  using V8 = typename E::vec8;
  constexpr int ROWB = fwd_row_bytes<D>();  // bytes per LDS row (D * 2 used)
  constexpr int EPB = fwd_epi_pitch<D>();   // bytes per row staged by the epilogue
  constexpr int GPR = D / 8;              // 16-byte granules of data per row
  constexpr int TILEB = kFwdBc * ROWB;    // bytes per tile buffer
  constexpr int NDMA = kFwdBc / kFwdWaves;  // V copies per wave per tile without VT (one per row)
  constexpr int NDMAK = GPR / kFwdWaves;     // K copies per wave per tile (dense rows)
  constexpr int NDMAV = D / (8 * kFwdWaves);  // V^T copies per wave per tile (8 rows each)
  constexpr int NDB = D / 32;             // output d-blocks of 32
  constexpr int KB = 0, VB = TILEB;       // buffer offsets
  constexpr int kKAhead = 3;              // K-fragment read-ahead, in d-steps
  constexpr int kVAhead = ACC16 ? (D > 512 ? 4 : 6) : 8;  // V-fragment read-ahead, in MFMAs
  // fp32 accumulator d-blocks that share the AGPRs with the Q fragments; the
  // remaining blocks live in VGPRs
  constexpr int kOAgpr = (256 - D / 4) / 16 < NDB ? (256 - D / 4) / 16 : NDB;

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- workgroup -> (b, h, q-tile)
  int t = xcd_logical(blockIdx.x, a.total_wg);
  int qt = t % a.n_qtiles;
  const int bh = t / a.n_qtiles;
  if (a.causal) qt = a.n_qtiles - 1 - qt;  // longest rows first
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int q0 = qt * kFwdRows;              // first row of the workgroup
  const int qw = q0 + wave * 32;             // first row of this wave
  const int my_q = qw + l32;                 // the row this lane accumulates

  const typename E::scalar* Q = (const typename E::scalar*)a.q + ((size_t)(b * a.Hq + h) * a.Nq) * D;
  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * a.Nkv) * D * 2;
  const uint32_t kv_bytes = (uint32_t)a.Nkv * D * 2;  // rows >= Nkv read as zeros
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc((const char*)a.k + kv_off, kv_bytes);
  // V: its transposed copy (VT), or V itself, staged like K
  const uint32_t vt_row = (uint32_t)a.nkv_pad * 2;  // bytes per row of V^T
  const __amdgpu_buffer_rsrc_t Vr =
      VT ? make_rsrc((const char*)a.vt + (size_t)(b * a.Hkv + hk) * D * a.nkv_pad * 2, (uint32_t)D * a.nkv_pad * 2)
         : make_rsrc((const char*)a.v + kv_off, kv_bytes);

  // ---- key range
  int kv_end = a.Nkv;
  if (a.causal) {
    int last_q = min(q0 + kFwdRows, a.Nq) - 1;
    kv_end = min(kv_end, last_q + 1);
  }
  const int n_tiles = (kv_end + kFwdBc - 1) / kFwdBc;

  // ---- stage the key bias [Nkv] in LDS (once; the host checks it fits),
  // zero-padded to whole tiles: keys >= Nkv are masked anyway. A per-query
  // mask [Nq, Nkv] is read from global memory, row by row, in the softmax.
  const bool has_mask = a.mask_rows > 0;
  const bool key_bias = a.bias_lds != 0;
  FFPA_LDS uint16_t* bias_lds = (FFPA_LDS uint16_t*)(smem + fwd_ring_bytes<D>());
  if (key_bias) {
    const uint16_t* mk = (const uint16_t*)a.mask;
    const int padded = ((a.Nkv + kFwdBc - 1) / kFwdBc) * kFwdBc;
    for (int i = threadIdx.x; i < padded; i += 256) bias_lds[i] = i < a.Nkv ? mk[i] : (uint16_t)0;
  }

  // ---- Q^T operand in registers: lane holds Q[my_q][16 s + 8 hi .. +7]
  u32x4 qf[D / 16];  // raw bits; kept in AGPRs as the B operand of the K-phase MFMAs
  {
    const int qrow = min(my_q, a.Nq - 1);
    const u32x4* qp = (const u32x4*)(Q + (size_t)qrow * D + 8 * hi);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qf[s] = qp[2 * s];
  }
  // compiler-visible: without it the K-phase MFMAs of every tile would wait
  // for the Q loads again, and those waits also hold for the copies in flight
  wait_vmcnt0_visible();
  __syncthreads();

  // ---- copy of one tile of K or V into its buffer. Copy instruction n of a
  // tile (n = wave + 4 r) fills LDS row n: lane i writes slot i, which holds
  // the logical granule i ^ swz4(n) of key row (64 tile + n). Granules past D
  // get an out-of-range offset and cost no memory traffic. The whole byte
  // offset goes in the per-lane offset, the part the buffer range check
  // covers, so that rows at or past Nkv read as zeros.
  auto issue_copy = [&](__amdgpu_buffer_rsrc_t rs, int buf, int tile, int r, int ln) {
    const int n = wave + kFwdWaves * r;
    const int lg = ln ^ swz4(n);
    const uint32_t lanepart = (GPR == 64 || lg < GPR) ? (uint32_t)lg << 4 : 0x80000000u;
    const uint32_t voff = lanepart + (uint32_t)(tile * kFwdBc + n) * (D * 2);
    dma16(rs, voff, smem + buf + n * ROWB);
  };
  auto issue_tile = [&](__amdgpu_buffer_rsrc_t rs, int buf, int tile) {
    int ln = lane;  // recomputed at each call rather than held across the loop
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int r = 0; r < NDMA; ++r) issue_copy(rs, buf, tile, r, ln);
  };
  // the copies of step st when a tile's NDMA copies are spread over the first
  // `span` steps of a phase
  auto issue_spread = [&](__amdgpu_buffer_rsrc_t rs, int buf, int tile, int st, int span, int ln) {
#pragma unroll
    for (int r = 0; r < NDMA; ++r)
      if ((r * span) / NDMA == st) issue_copy(rs, buf, tile, r, ln);
  };
  // ---- copy of one K tile as 64 dense rows of GPR granules (dense_pos):
  // copy instruction n (n = wave + 4 r, r < GPR / 4) fills slots 64 n + lane
  // of the tile, slot s holding granule dense_pos(GPR, row, s % GPR) of row
  // s / GPR. Every instruction carries a full 1 KiB, which matters below
  // D = 512: the copy path costs per instruction, not per byte.
  auto k_copy = [&](int tile, int r, int ln) {
    if constexpr (GPR == 64) {
      issue_copy(Kr, KB, tile, r, ln);  // one row per instruction: the same layout
    } else {
      const int n = wave + kFwdWaves * r;
      const int sl = 64 * n + ln;
      const int row = sl / GPR, g = dense_pos(GPR, row, sl % GPR);
      const uint32_t voff = (uint32_t)(g << 4) + (uint32_t)(tile * kFwdBc + row) * (D * 2);
      dma16(Kr, voff, smem + KB + n * 1024);
    }
  };
  auto issue_k_tile = [&](int tile) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int r = 0; r < NDMAK; ++r) k_copy(tile, r, ln);
  };
  auto issue_spread_k = [&](int tile, int st, int span, int ln) {
#pragma unroll
    for (int r = 0; r < NDMAK; ++r)
      if ((r * span) / NDMAK == st) k_copy(tile, r, ln);
  };
  // ---- copy of one V^T tile (D rows of 64 keys = 128 bytes). Copy
  // instruction n (n = wave + 4 r) fills LDS rows 8 n .. 8 n + 7: lane i
  // writes slot i % 8 of row 8 n + i / 8, which holds the logical granule
  // (positions 8 g .. 8 g + 7) g = (i % 8) ^ vt_swz(row), vt_swz(row) =
  // (row / 2) % 8. Within the 8 rows of one instruction vt_swz = 4 (n % 2) +
  // (i / 8) / 2, so the per-lane part of the offset takes one of two values,
  // by n's parity.
  auto vt_lane_offsets = [&](int ln, uint32_t* lo) {
    const int rl = ln >> 3;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      lo[par] = (uint32_t)rl * vt_row + (uint32_t)(((ln & 7) ^ (rl >> 1) ^ (4 * par)) << 4);
  };
  auto issue_spread_v = [&](int tile, int st, int span, const uint32_t* lo) {
#pragma unroll
    for (int r = 0; r < NDMAV; ++r)
      if ((r * span) / NDMAV == st) {
        const int n = wave + kFwdWaves * r;
        const uint32_t voff = lo[n & 1] + (uint32_t)(8 * n) * vt_row + (uint32_t)tile * (kFwdBc * 2);
        dma16(Vr, voff, smem + VB + n * 1024);
      }
  };
  // the V copies of either layout: per-lane setup, then the copies of step st
  auto v_lane_offsets = [&](int ln, uint32_t* lo) {
    if constexpr (VT) vt_lane_offsets(ln, lo);
    else lo[0] = (uint32_t)ln;
  };
  auto v_copy_spread = [&](int tile, int st, int span, const uint32_t* lo) {
    if constexpr (VT) issue_spread_v(tile, st, span, lo);
    else issue_spread(Vr, VB, tile, st, span, (int)lo[0]);
  };

  // ---- LDS read addresses: per-lane bases (recomputed at the start of each
  // phase, so they are live only there) plus compile-time offsets < 64 KiB.
  // K fragment (A of S^T) for d-step s = 8 a + c: row 32 kb + l32, logical
  // granule 16 a + 2 c + hi, stored at 16 a + dense_pos(row, 2 c + hi) (the
  // swizzle groups divide 16, and rows 32 apart swizzle alike).
  auto k_bases = [&](int ln, uint32_t* kx) {
    const int r = ln & 31, h = ln >> 5;
#pragma unroll
    for (int c = 0; c < 8; ++c) kx[c] = (uint32_t)(KB + r * (GPR * 16) + (dense_pos(GPR, r, 2 * c + h) << 4));
  };
  auto k_addr = [&](const uint32_t* kx, int st, int kb) -> uint32_t {
    return kx[st & 7] + 256 * (st >> 3) + 32 * kb * (GPR * 16);
  };
  // V^T fragment (A of O^T) for d-block db and the 16-key step (kb, t2):
  // row 32 db + l32 of the V^T tile, logical granule 4 kb + 2 t2 + hi, whose
  // 8 positions hold the keys the lane's P operand pairs with (vt_key).
  // Sixteen consecutive lanes read sixteen consecutive rows: two rows share a
  // 256-byte bank window, and (row / 2) % 8 spreads the pairs over it.
  //
  // Without the transposed copy (!VT), V is staged like K and V^T fragments
  // come from transposed reads: group G = lane/16, i = lane%16 reads row
  // 32 kb + 16 t2 + 8 r8 + 4 (G/2) + i/4 at columns 32 db + 16 (G%2) + 4 (i%4),
  // i.e. logical granule 4 db + y with y = 2 (G%2) + (i%4)/2, at half the LDS
  // byte rate of 16-byte reads. The host takes this layout when the problem
  // has too few queries per key to repay the transposition pass.
  auto v_bases = [&](int ln, uint32_t* vx) {
    if constexpr (VT) {
      const int r = ln & 31, h = ln >> 5, x = (r >> 1) & 7;
#pragma unroll
      for (int p = 0; p < 4; ++p) vx[p] = (uint32_t)(VB + r * 128 + (((2 * p + h) ^ x) << 4));
    } else {
      const int G = ln >> 4, gi = ln & 15;
      const int vrow = 4 * (G >> 1) + (gi >> 2);
      const int y = 2 * (G & 1) + ((gi & 3) >> 1);
#pragma unroll
      for (int r8 = 0; r8 < 2; ++r8) {
        const int row = vrow + 8 * r8, x = swz4(row);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vx[4 * r8 + e] = (uint32_t)(VB + row * ROWB + (((4 * e + y) ^ x) << 4) + (gi & 1) * 8);
      }
    }
  };
  auto v_read = [&](const uint32_t* vx, int db, int kb, int t2) -> u32x4 {
    if constexpr (VT) {
      return lds_read16(smem + vx[2 * kb + t2] + 4096 * db);
    } else {
      const uint32_t off = 256 * (db >> 2) + (32 * kb + 16 * t2) * ROWB;
      return join8(lds_read_tr(smem + vx[db & 3] + off), lds_read_tr(smem + vx[4 + (db & 3)] + off));
    }
  };

  // ---- accumulators
  f32x16 o_acc[ACC16 ? 1 : NDB];
  u32x4 o16[ACC16 ? NDB * 2 : 1];  // fp16 pairs: d-block db uses o16[2db], o16[2db+1]
  if constexpr (!ACC16) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) o_acc[i] = f32x16{};
  } else {
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) o16[i] = u32x4{0, 0, 0, 0};
  }
  float m_ref = -INFINITY;  // reference max (log2 domain)
  float l_run = 0.f;        // ACC32: this lane's partial row sum; ACC16: full row sum
  bool fresh = true;        // ACC32: no PV product accumulated yet
  bool safe = false;        // ACC32: a tile broke m_ref + tau; the key loop reruns per tile
  // dropout of 16 scores of row q held by a lane, keys k0 + 8 g + e (g, e in
  // 0..3; k0 a multiple of 4): the quad's four generator calls, one a lane
  auto drop_half = [&](float* tv, int k0, int q) {
    const uint32_t keep = drop_bits_row(a.drop, b * a.Hq + h, q, k0);
#pragma unroll
    for (int i = 0; i < 16; ++i) tv[i] = keep_if_bit(tv[i], keep, i);
  };
  // one word per wave: did a row of that wave break m_ref + tau in this tile
  FFPA_LDS uint32_t* restart_flag = (FFPA_LDS uint32_t*)(smem + fwd_ring_bytes<D>() +
                                                         (key_bias ? fwd_bias_bytes(a.Nkv) : 0));

  if constexpr (!ACC16) {
    // ---- fp32 accumulation. A tile's scores are two 32-key halves, each one
    // MFMA chain over D. The softmax of half 0 runs beside the chain of half
    // 1, and the softmax of half 1 beside the P V products of half 0, so the
    // matrix cores do not wait for the exponentials. The restart test of a
    // tile (some row above m_ref + tau) is read after the next tile's first
    // barrier: the tile that broke the bound has been accumulated by then,
    // which the restart discards with everything else.
    constexpr int NS = D / 16;        // d-steps of one chain
    constexpr int kKA = 6;            // K fragments read ahead
    float mx_prev = -INFINITY;        // the previous tile's row max (log2 domain)
    issue_k_tile(0);
    for (int j = 0; j <= n_tiles; ++j) {
      const int j0 = j * kFwdBc;
      int lj = lane;
      asm volatile("" : "+v"(lj));
      const int hij = lj >> 5;
      const int my_qj = qw + (lj & 31);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        if (d < kOAgpr) asm volatile("" : "+a"(o_acc[d]));
        else asm volatile("" : "+v"(o_acc[d]));
      }
      wait_vmcnt<0>();  // K(j) landed (this wave's copies) ...
      wait_lgkm0();
      barrier();        // ... and everyone's; everyone is done with V(j-1)
      if (j > 0) {
        const u32x4 f = *(const FFPA_LDS u32x4*)restart_flag;
        if ((f[0] | f[1] | f[2] | f[3]) != 0) {  // workgroup-uniform
          // the rest runs in the per-tile loop below, from the first tile,
          // with the raised reference: no tile can force a second pass
          m_ref = fmaxf(m_ref, mx_prev);
          safe = true;
          break;
        }
      }
      if (j == n_tiles) break;

      const bool need_mask = has_mask || (j0 + kFwdBc > a.Nkv) || (a.causal && j0 + kFwdBc - 1 > qw);
      const int kb0 = j0 + 4 * hij;  // lane's keys: kb0 + 32 kb + 8 (i / 4) + i % 4
      // scaled (and masked) scores of half kb in the log2 domain, and their
      // row max over the half
      auto half_scores = [&](const f32x16& s, int kb, float* tv) -> float {
#pragma unroll
        for (int i = 0; i < 16; ++i) tv[i] = s[i] * a.scale_log2;
        if (need_mask) {
          if (has_mask && !key_bias) {
            const uint16_t* mrow = (const uint16_t*)a.mask + (size_t)min(my_qj, a.Nq - 1) * a.mask_stride;
            const bool by8 = (a.Nkv & 3) == 0;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const f32x4 bv = mask_row4<BF16>(mrow, kb0 + 32 * kb + 8 * g4, a.Nkv, by8);
#pragma unroll
              for (int e = 0; e < 4; ++e) tv[4 * g4 + e] += bv[e] * kLog2e;
            }
          }
          if (key_bias) {
            const FFPA_LDS char* bp = (const FFPA_LDS char*)bias_lds + 2 * (kb0 + 32 * kb);
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const u32x2 w = *(const FFPA_LDS u32x2*)(bp + 16 * g4);
              tv[4 * g4 + 0] += E::to_f32((uint16_t)(w[0] & 0xffff)) * kLog2e;
              tv[4 * g4 + 1] += E::to_f32((uint16_t)(w[0] >> 16)) * kLog2e;
              tv[4 * g4 + 2] += E::to_f32((uint16_t)(w[1] & 0xffff)) * kLog2e;
              tv[4 * g4 + 3] += E::to_f32((uint16_t)(w[1] >> 16)) * kLog2e;
            }
          }
          int klim = a.Nkv - kb0 - 32 * kb;
          if (a.causal) klim = min(klim, my_qj + 1 - kb0 - 32 * kb);
#pragma unroll
          for (int i = 0; i < 16; ++i) tv[i] = (8 * (i >> 2) + (i & 3)) >= klim ? -INFINITY : tv[i];
        }
        float mh = tv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mh = fmaxf(mh, tv[i]);
        mh = fmaxf(mh, swap_halves(mh));
        // first unmasked keys of this row: adopt their max (O and l are still 0)
        if (m_ref == -INFINITY) m_ref = mh;
        return mh;
      };
      // P = 2^(t - m_ref) of elements [i0, i1) of a half, summed into l_run
      auto half_exp = [&](float* tv, int i0, int i1) {
        const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
#pragma unroll
        for (int i = i0; i < i1; ++i) {
          tv[i] = exp2_fast(tv[i] - m_use);
          l_run += tv[i];
        }
      };
      // the MFMA operand P of half kb: dropout zeroes the dropped elements
      // here (the row sum has the undropped ones); the scale of the kept ones
      // is applied to O at the end
      auto half_pack = [&](float* tv, V8* pf, int kb) {
        if constexpr (DROP) drop_half(tv, j0 + 4 * hij + 32 * kb, my_qj);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const float* x = &tv[8 * t2];
          pf[t2] = pack8<BF16>(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
        }
      };
      // softmax work of a half spread over the NS MFMA slots q = 0 .. NS - 1
      // beside it: the scores at slot 0, the exponentials of element i at
      // slot 1 + i (NS - 2) / 16, the packing after the last one. Each
      // element is pinned at its slot, so the compiler keeps the order.
      auto half_slot = [&](const f32x16& s, int kb, int q, float* tv, float& mh, V8* pf) {
        if (q == 0) mh = half_scores(s, kb, tv);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int slot = NS > 2 ? 1 + (i * (NS - 2)) / 16 : NS - 1;
          if (slot == q) {
            asm volatile("" : "+v"(tv[i]));
            half_exp(tv, i, i + 1);
          }
        }
        if (q == NS - 1) {
          half_pack(tv, pf, kb);
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(pf[t2]));
        }
      };

      // ===== K phase: S^T = K Q^T, half 0 then half 1, with the softmax of
      // half 0 beside the chain of half 1. The copies of V(j) are spread over
      // the chain of half 0.
      f32x16 s_acc[2];
      float tv0[16], tv1[16];
      float mh0 = -INFINITY, mh1 = -INFINITY;
      V8 pf0[2], pf1[2];
      {
        u32x4 kf[kKA];
        uint32_t kx[8];
        k_bases(lj, kx);
        auto kread = [&](int c) { return lds_read16(smem + k_addr(kx, c % NS, c / NS)); };
#pragma unroll
        for (int c = 0; c < kKA; ++c) kf[c] = kread(c);
        uint32_t vlo[2];
        {
          int lnc = lane;
          asm volatile("" : "+v"(lnc));
          v_lane_offsets(lnc, vlo);
        }
#pragma unroll
        for (int c = 0; c < 2 * NS; ++c) {
          v_copy_spread(j, c, NS, vlo);
          const u32x4 a0 = kf[c % kKA];
          if (c + kKA < 2 * NS) kf[c % kKA] = kread(c + kKA);
          const int st = c % NS;
          f32x16& acc = s_acc[c / NS];
          // each chain ends padded for the VALU that reads its scores next
          if (st == 0) mfma32_asm<BF16, true, false, true>(acc, a0, qf[st]);
          else if (st == NS - 1) mfma32_asm<BF16, true, false, false, false, true>(acc, a0, qf[st]);
          else mfma32_asm<BF16, true, false>(acc, a0, qf[st]);
          if (c == NS - 1) pin_after_pad(s_acc[0]);
          if (c >= NS) half_slot(s_acc[0], 0, c - NS, tv0, mh0, pf0);
        }
        pin_after_pad(s_acc[1]);
      }

      // ===== V phase: O^T += V^T P^T
      wait_vmcnt<0>();  // V(j) landed ...
      wait_lgkm0();
      barrier();        // ... everywhere; everyone is done with K(j)
      // The P V products, as a lambda instantiated for the first tile of an
      // attempt (FRESH: the first product of each block starts from C = 0) and
      // for the others, so that no MFMA of the hot loop sits behind a branch.
      // Step st = NDB p + db, p = 2 kb + t2: the products of half 0 come
      // first, and the softmax of half 1 runs beside them.
      auto v_phase = [&](auto fresh_tag) {
        constexpr bool FRESH = decltype(fresh_tag)::value;
        constexpr int NSV = 4 * NDB;
        uint32_t vx[8];
        {
          int lv = lane;
          asm volatile("" : "+v"(lv));
          v_bases(lv, vx);
        }
        auto vread = [&](int st) {
          const int p = st / NDB, db = st % NDB;
          return v_read(vx, db, p >> 1, p & 1);
        };
        u32x4 vf[kVAhead];
#pragma unroll
        for (int st = 0; st < kVAhead; ++st) vf[st] = vread(st);
        int lnc = lane;
        asm volatile("" : "+v"(lnc));
#pragma unroll
        for (int st = 0; st < NSV; ++st) {
          // on the last tile this copies rows past the key range (range-checked
          // zeros) or, causal, rows nobody reads: harmless, and branch-free
          issue_spread_k(j + 1, st, NSV / 2, lnc);
          const int p = st / NDB, db = st % NDB;
          const int kb = p >> 1, t2 = p & 1;
          const u32x4 vbits = vf[st % kVAhead];
          if (st + kVAhead < NSV) vf[st % kVAhead] = vread(st + kVAhead);
          const u32x4 pb = __builtin_bit_cast(u32x4, kb == 0 ? pf0[t2] : pf1[t2]);
          // the first MFMA of each half pads for the VALU that wrote its P;
          // the last one pads for accumulator copies on the loop's edges
          const bool first = st == 0 || st == 2 * NDB;
          const bool zero = FRESH && p == 0;
          const bool pad_after = st == NSV - 1;
          if (db < kOAgpr) {
            if (zero) {
              if (first) mfma32_asm<BF16, false, true, true, true>(o_acc[db], vbits, pb);
              else mfma32_asm<BF16, false, true, true>(o_acc[db], vbits, pb);
            } else if (first) {
              mfma32_asm<BF16, false, true, false, true>(o_acc[db], vbits, pb);
            } else if (pad_after) {
              mfma32_asm<BF16, false, true, false, false, true>(o_acc[db], vbits, pb);
            } else {
              mfma32_asm<BF16, false, true>(o_acc[db], vbits, pb);
            }
          } else {
            if (zero) {
              if (first) mfma32_asm<BF16, false, false, true, true>(o_acc[db], vbits, pb);
              else mfma32_asm<BF16, false, false, true>(o_acc[db], vbits, pb);
            } else if (first) {
              mfma32_asm<BF16, false, false, false, true>(o_acc[db], vbits, pb);
            } else if (pad_after) {
              mfma32_asm<BF16, false, false, false, false, true>(o_acc[db], vbits, pb);
            } else {
              mfma32_asm<BF16, false, false>(o_acc[db], vbits, pb);
            }
          }
          // softmax of half 1 over the first NS products (2 NDB >= NS)
          if (st < NS) half_slot(s_acc[1], 1, st, tv1, mh1, pf1);
          if (st == NS - 1) {
            // restart test of the tile, read after the next tile's first barrier
            float mx = fmaxf(mh0, mh1);
            mx_prev = mx;
            const bool broke = mx > m_ref + fwd_tau<BF16>();
            const uint32_t any_broke = __builtin_amdgcn_ballot_w64(broke) != 0 ? 1u : 0u;
            if (lane == 0) restart_flag[wave] = any_broke;
          }
        }
      };
      if (fresh) v_phase(BoolTag<true>{});
      else v_phase(BoolTag<false>{});
      fresh = false;
    }
  }
  // ---- the per-tile loop: the fp16 accumulator (renormalised every tile),
  // and with fp32 accumulation the safe mode after a tile broke the bound
  // (P of a tile computed from the raised reference before its products;
  // O rescaled when the reference rises by more than tau). Its score and
  // product phases run one after the other.
  if (ACC16 || safe) {
  if constexpr (!ACC16) {
    // the fast loop's copies in flight land before the buffers are reused;
    // O and l start over
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
#pragma unroll
    for (int d = 0; d < NDB; ++d) o_acc[d] = f32x16{};
    l_run = 0.f;
  }
  issue_k_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    const int j0 = j * kFwdBc;
    // per-lane values are re-derived from the lane id in each iteration (one
    // live VGPR instead of several across the loop)
    int lj = lane;
    asm volatile("" : "+v"(lj));
    const int hij = lj >> 5;
    const int my_qj = qw + (lj & 31);
    if constexpr (!ACC16) {
#pragma unroll
      for (int d = 0; d < NDB; ++d) {
        if (d < kOAgpr) asm volatile("" : "+a"(o_acc[d]));
        else asm volatile("" : "+v"(o_acc[d]));
      }
    }
    // ===== K phase: S^T = K Q^T
    wait_vmcnt<0>();  // K(j) landed (this wave's copies) ...
    wait_lgkm0();
    barrier();        // ... and everyone's; everyone is done with V(j-1)
    // The copies of V(j) are spread over the first half of the phase's MFMAs
    // (issue_spread), which keeps their LDS writes from piling up at once.
    f32x16 s_acc[2];
    {
      // K fragments are read kKAhead d-steps ahead of the MFMAs that use them
      constexpr int NS = D / 16;
      u32x4 kf[kKAhead][2];
      uint32_t kx[8];
      k_bases(lj, kx);
      auto kread = [&](int st, int kb) { return lds_read16(smem + k_addr(kx, st, kb)); };
#pragma unroll
      for (int st = 0; st < kKAhead; ++st) {
        kf[st][0] = kread(st, 0);
        kf[st][1] = kread(st, 1);
      }
      uint32_t vlo[2];
      {
        int lnc = lane;
        asm volatile("" : "+v"(lnc));
        v_lane_offsets(lnc, vlo);
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        v_copy_spread(j, st, NS > 1 ? NS / 2 : 1, vlo);
        const u32x4 a0 = kf[st % kKAhead][0], a1 = kf[st % kKAhead][1];
        if (st + kKAhead < NS) {
          kf[st % kKAhead][0] = kread(st + kKAhead, 0);
          kf[st % kKAhead][1] = kread(st + kKAhead, 1);
        }
        // S^T chains in VGPRs, Q operand from AGPRs; the last pair pads for the
        // softmax VALU that reads the scores next
        if (st == 0) {
          mfma32_asm<BF16, true, false, true>(s_acc[0], a0, qf[st]);
          mfma32_asm<BF16, true, false, true>(s_acc[1], a1, qf[st]);
        } else if (st == NS - 1) {
          mfma32_asm<BF16, true, false, false>(s_acc[0], a0, qf[st]);
          mfma32_asm<BF16, true, false, false, false, true>(s_acc[1], a1, qf[st]);
          pin_after_pad(s_acc[0]);
        } else {
          mfma32_asm<BF16, true, false>(s_acc[0], a0, qf[st]);
          mfma32_asm<BF16, true, false>(s_acc[1], a1, qf[st]);
        }
      }
    }

    // ===== online softmax on the tile (log2 domain)
    const bool need_mask = has_mask || (j0 + kFwdBc > a.Nkv) ||
                           (a.causal && j0 + kFwdBc - 1 > qw);
    float tv[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tv[kb][i] = s_acc[kb][i] * a.scale_log2;
    if (need_mask) {
      // lane's keys: j0 + 4 hi + c, c = 32 kb + 8 (i / 4) + i % 4
      const int kb0 = j0 + 4 * hij;
      if (has_mask && !key_bias) {
        // mask from global memory: row my_q (clamped to the last row) of a
        // per-query mask, or the key bias when it is not staged; four
        // consecutive keys per group
        const uint16_t* mrow = (const uint16_t*)a.mask + (size_t)min(my_qj, a.Nq - 1) * a.mask_stride;
        const bool by8 = (a.Nkv & 3) == 0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 bv = mask_row4<BF16>(mrow, kb0 + 32 * kb + 8 * g4, a.Nkv, by8);
#pragma unroll
            for (int e = 0; e < 4; ++e) tv[kb][4 * g4 + e] += bv[e] * kLog2e;
          }
      }
      if (key_bias) {
        // additive bias, four consecutive keys per 8-byte LDS read
        const FFPA_LDS char* bp = (const FFPA_LDS char*)bias_lds + 2 * kb0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const u32x2 w = *(const FFPA_LDS u32x2*)(bp + 2 * (32 * kb + 8 * g4));
            tv[kb][4 * g4 + 0] += E::to_f32((uint16_t)(w[0] & 0xffff)) * kLog2e;
            tv[kb][4 * g4 + 1] += E::to_f32((uint16_t)(w[0] >> 16)) * kLog2e;
            tv[kb][4 * g4 + 2] += E::to_f32((uint16_t)(w[1] & 0xffff)) * kLog2e;
            tv[kb][4 * g4 + 3] += E::to_f32((uint16_t)(w[1] >> 16)) * kLog2e;
          }
      }
      // keys at or past the limit are dead: past Nkv, or after this row (causal)
      int klim = a.Nkv - kb0;
      if (a.causal) klim = min(klim, my_qj + 1 - kb0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int c = 32 * kb + 8 * (i >> 2) + (i & 3);
          tv[kb][i] = c >= klim ? -INFINITY : tv[kb][i];
        }
    }
    float mx = tv[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, tv[kb][i]);
    mx = fmaxf(mx, swap_halves(mx));

    float alpha = 1.f;
    {
      const bool need = mx > m_ref + (ACC16 ? kRescaleTau : fwd_tau<BF16>());
      if (__builtin_amdgcn_ballot_w64(need) != 0) {  // wave-uniform branch
        const float m_new = fmaxf(m_ref, mx);
        alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_ref - m_new);
        m_ref = m_new;
        if constexpr (!ACC16) {
          // fp32 O follows the raised reference; the pins keep the products
          // of this tile behind the rescale
#pragma unroll
          for (int d = 0; d < NDB; ++d) {
            if (d < kOAgpr) {
              scale_agpr16(o_acc[d], alpha);
              asm volatile("" : "+a"(o_acc[d]));
            } else {
              o_acc[d] *= alpha;
              asm volatile("" : "+v"(o_acc[d]));
            }
          }
        }
      }
    }
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        tv[kb][i] = exp2_fast(tv[kb][i] - m_use);
        psum += tv[kb][i];
      }
    // fp16: normalised accumulator, O <- O * (alpha l_old / l_new) + (P / l_new) V;
    // fp32: O <- alpha O + P V, this lane's partial sum as in the fast loop
    float pscale = 1.f, oscale = 1.f;
    if constexpr (ACC16) {
      const float l_old = l_run;
      const float l_new = alpha * l_old + psum + swap_halves(psum);
      l_run = l_new;
      pscale = l_new > 0.f ? 1.f / l_new : 0.f;
      oscale = alpha * l_old * pscale;
    } else {
      l_run = alpha * l_run + psum;
    }
    V8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        if constexpr (DROP)
          if (t2 == 0) drop_half(tv[kb], j0 + 4 * hij + 32 * kb, my_qj);
        const float* x = &tv[kb][8 * t2];
        if constexpr (ACC16)
          pf[kb][t2] = pack8<BF16>(x[0] * pscale, x[1] * pscale, x[2] * pscale, x[3] * pscale,
                                   x[4] * pscale, x[5] * pscale, x[6] * pscale, x[7] * pscale);
        else
          pf[kb][t2] = pack8<BF16>(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
      }

    // P is the B operand of MFMAs issued as inline asm, which the compiler
    // does not pad for hazards: force every VALU write of P to happen here,
    // before the barrier (the first MFMA of the phase also pads).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(pf[kb][t2]));

    // ===== V phase: O^T += V^T P^T
    wait_vmcnt<0>();  // V(j) landed ...
    wait_lgkm0();
    barrier();        // ... everywhere; everyone is done with K(j)
    {
      // Step order: consecutive MFMAs write different accumulators (a
      // dependent MFMA waits for its predecessor's result). fp16: d-blocks go
      // in pairs, each with a per-tile product in VGPRs: st = 8 q + 2 p +
      // side, db = 2 q + side, p = 2 kb + t2 the (key block, k-step) pair.
      // fp32: st = NDB p + db. V^T fragments are read kVAhead MFMAs ahead of
      // their use.
      constexpr int NSV = 4 * NDB;
      auto step = [](int st, int& db, int& kb, int& t2) {
        int p;
        if constexpr (ACC16) {
          p = (st & 7) >> 1;
          db = 2 * (st >> 3) + (st & 1);
        } else {
          p = st / NDB;
          db = st % NDB;
        }
        kb = p >> 1;
        t2 = p & 1;
      };
      uint32_t vx[8];
      {
        int lv = lane;
        asm volatile("" : "+v"(lv));
        v_bases(lv, vx);
      }
      auto vread = [&](int st) {
        int db, kb, t2;
        step(st, db, kb, t2);
        return v_read(vx, db, kb, t2);
      };
      u32x4 vf[kVAhead];
#pragma unroll
      for (int st = 0; st < kVAhead; ++st) vf[st] = vread(st);
      // fp16 path: per-tile products of a pair's even / odd block, two sets
      // (pairs alternate): the fold of pair q into the fp16 accumulator runs
      // beside the products of pair q + 1
      f32x16 acc_e[2], acc_o[2];
      // o16 <- o16 * oscale + acc, in packed fp16, for half hh of block d2
      auto fold_half = [&](const f32x16& acc, int d2, int hh) {
        const f16x2 sc = {(_Float16)oscale, (_Float16)oscale};
        u32x4 w = o16[2 * d2 + hh];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f16x2 cur = f16x2_from_bits(w[e]);
          const f16x2 add = {(_Float16)acc[8 * hh + 2 * e], (_Float16)acc[8 * hh + 2 * e + 1]};
          cur = cur * sc + add;
          w[e] = __builtin_bit_cast(uint32_t, cur);
        }
        o16[2 * d2 + hh] = w;
      };
      auto fold = [&](const f32x16& acc, int d2) {
        fold_half(acc, d2, 0);
        fold_half(acc, d2, 1);
      };
      int lnc = lane;
      asm volatile("" : "+v"(lnc));
#pragma unroll
      for (int st = 0; st < NSV; ++st) {
        // on the last tile this copies rows past the key range (range-checked
        // zeros) or, causal, rows nobody reads: harmless, and branch-free
        issue_spread_k(j + 1, st, NSV / 2, lnc);
        int db, kb, t2;
        step(st, db, kb, t2);
        const u32x4 vbits = vf[st % kVAhead];
        if (st + kVAhead < NSV) vf[st % kVAhead] = vread(st + kVAhead);
        const u32x4 pb = __builtin_bit_cast(u32x4, pf[kb][t2]);
        const bool first = kb == 0 && t2 == 0;
        const bool final_mfma = st == NSV - 1;
        if constexpr (ACC16) {
          // per-tile products in VGPRs, set q % 2 for pair q = st / 8; the
          // last pair's last MFMA pads for the fold after the loop
          const int q = st >> 3, set = q & 1;
          if ((st & 1) == 0) {
            if (first) {
              if (st == 0) mfma32_asm<BF16, false, false, true, true>(acc_e[set], vbits, pb);
              else mfma32_asm<BF16, false, false, true>(acc_e[set], vbits, pb);
            } else {
              mfma32_asm<BF16, false, false>(acc_e[set], vbits, pb);
            }
          } else {
            if (first) mfma32_asm<BF16, false, false, true>(acc_o[set], vbits, pb);
            else if (final_mfma) mfma32_asm<BF16, false, false, false, false, true>(acc_o[set], vbits, pb);
            else mfma32_asm<BF16, false, false>(acc_o[set], vbits, pb);
          }
          // pair q - 1 folds at steps 6 (even block) and 7 (odd block) of
          // pair q: seven MFMAs of pair q have issued since its last one
          if (q > 0 && (st & 7) == 6) {
            pin_after_pad(acc_e[set ^ 1]);
            pin_after_pad(acc_o[set ^ 1]);
            fold(acc_e[set ^ 1], 2 * (q - 1));
          }
          if (q > 0 && (st & 7) == 7) fold(acc_o[set ^ 1], 2 * (q - 1) + 1);
          if (final_mfma) {
            pin_after_pad(acc_e[set]);
            fold(acc_e[set], 2 * q);
            fold(acc_o[set], 2 * q + 1);
          }
        } else {
          // fp32 O accumulates in place (zeroed before the loop); the first
          // MFMA pads for the VALU that wrote P (and a rescale), the last for
          // whatever reads the accumulators after the phase
          if (db < kOAgpr) {
            if (st == 0) mfma32_asm<BF16, false, true, false, true>(o_acc[db], vbits, pb);
            else if (final_mfma) mfma32_asm<BF16, false, true, false, false, true>(o_acc[db], vbits, pb);
            else mfma32_asm<BF16, false, true>(o_acc[db], vbits, pb);
          } else {
            if (st == 0) mfma32_asm<BF16, false, false, false, true>(o_acc[db], vbits, pb);
            else if (final_mfma) mfma32_asm<BF16, false, false, false, false, true>(o_acc[db], vbits, pb);
            else mfma32_asm<BF16, false, false>(o_acc[db], vbits, pb);
          }
        }
      }
    }
  }
  }
  wait_vmcnt<0>();  // no copy may still target this workgroup's LDS when it ends
  if constexpr (!ACC16) {
    // the accumulators were last written by MFMAs issued as inline asm: pad
    // before the epilogue reads them (the padding is tied to every block)
    asm volatile("s_nop 7\n s_nop 7\n s_nop 4" ::: "memory");
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      if (d < kOAgpr) asm volatile("" : "+a"(o_acc[d]));
      else asm volatile("" : "+v"(o_acc[d]));
    }
  }

  // ===== epilogue: normalise, store O and lse
  // The accumulators hold O transposed (a lane has 4-element pieces of one
  // row), so the rows go through LDS first: each wave writes its 32 rows to a
  // slice of the (now idle) tile buffers (32 rows of EPB bytes), then stores
  // them as one contiguous run of 32 D elements. Written straight from the
  // accumulators, a cache line of O would be filled by many partial writes and
  // leave the L2 several times.
  int le = threadIdx.x & 63;
  asm volatile("" : "+v"(le));  // derived afresh: no lane value lives across the loop
  const int hie = le >> 5, my_qe = qw + (le & 31);
  float l_tot, inv;
  if constexpr (!ACC16) {
    l_tot = l_run + swap_halves(l_run);
    inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if constexpr (DROP) inv *= a.drop.scale;
  } else {
    l_tot = l_run;
    inv = 1.f;
  }
  wait_lgkm0();
  barrier();  // every wave is done reading the tile buffers
  FFPA_LDS char* ostage = smem + wave * 32 * EPB;
  {
    // row r = lane % 32 of the wave; granule g (8 elements) sits in slot
    // g ^ (r % 16), which puts 16 consecutive rows on distinct banks
    const int r = le & 31;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float x0, x1, x2, x3;
        if constexpr (!ACC16) {
          x0 = o_acc[db][4 * g4 + 0] * inv;
          x1 = o_acc[db][4 * g4 + 1] * inv;
          x2 = o_acc[db][4 * g4 + 2] * inv;
          x3 = o_acc[db][4 * g4 + 3] * inv;
        } else {
          const u32x4 w = o16[2 * db + (g4 >> 1)];
          const f16x2 p0 = f16x2_from_bits(w[2 * (g4 & 1)]);
          const f16x2 p1 = f16x2_from_bits(w[2 * (g4 & 1) + 1]);
          x0 = (float)p0[0];
          x1 = (float)p0[1];
          x2 = (float)p1[0];
          x3 = (float)p1[1];
        }
        const u32x2 st = {E::pack2(x0, x1), E::pack2(x2, x3)};
        const int g = 4 * db + g4;  // elements 32 db + 8 g4 + 4 hi .. +3
        *(FFPA_LDS u32x2*)(ostage + r * EPB + ((g ^ (r & 15)) << 4) + 8 * hie) = st;
      }
    }
  }
  // a wave's LDS accesses complete in order: its own rows can be read back
  // without a barrier. The wave's 32 rows are one contiguous run of O.
  {
    typename E::scalar* O = (typename E::scalar*)a.o + ((size_t)(b * a.Hq + h) * a.Nq + qw) * D;
    const int rows = min(32, a.Nq - qw);
#pragma unroll
    for (int it = 0; it < GPR / 2; ++it) {
      const int c = it * 64 + le;  // granule index within the wave's rows
      const int r = c / GPR, g = c % GPR;
      const u32x4 x = *(const FFPA_LDS u32x4*)(ostage + r * EPB + ((g ^ (r & 15)) << 4));
      if (r < rows) *(u32x4*)(O + (size_t)c * 8) = x;
    }
  }
  if (my_qe < a.Nq && a.lse != nullptr && hie == 0) {
    float* L = a.lse + (size_t)(b * a.Hq + h) * a.Nq + my_qe;
    *L = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

// Host launcher. lds_bytes = tile buffers + key-bias bytes [+ restart flags]
// (the caller checks <= 160 KiB); above D = 512 the launch takes at least the
// epilogue's staging, which is larger than the tiles. With VT the transposed copy of V is written into a.vt first.
// The kernel's LDS limit is set before anything is enqueued, so a failure
// there leaves the stream untouched.
template <int D, bool BF16, bool ACC16, bool VT, bool DROP = false>
hipError_t launch_fwd_prefill(const FwdArgs& a, size_t lds_bytes, hipStream_t stream) {
  auto kern = fwd_prefill_kernel<D, BF16, ACC16, VT, DROP>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  if constexpr (VT) {
    const hipError_t e = launch_fwd_vt(a.v, const_cast<void*>(a.vt), a.B * a.Hkv, a.Nkv, D, a.nkv_pad, stream);
    if (e != hipSuccess) return e;
  }
  const size_t lds = lds_bytes > (size_t)fwd_epi_bytes<D>() ? lds_bytes : (size_t)fwd_epi_bytes<D>();
  hipLaunchKernelGGL(kern, dim3(a.total_wg), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
