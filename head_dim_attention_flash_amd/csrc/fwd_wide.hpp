// Forward attention for head dimensions above 512 (multiples of 64 up to 1024).
//
// Same operation as fwd_prefill.hpp: O = softmax(scale * Q K^T + mask) V and
// lse per row (the "naive_math" definition of section 3 of the
// attention-kernel-profiler design document; mask and GQA conventions of
// "FFPA Attention Benchmark", "Quick Start", and the profiler's "gqa_4kv").
// The D sweep of that benchmark page runs to D = 1024.
//
// At D = 1024 one wave cannot hold both the Q fragments and the fp32 output
// accumulators of 32 rows (256 + 512 registers). So D is split in two halves
// inside the workgroup: 4 waves = 2 row blocks of 32 queries x 2 halves of D.
// A wave keeps Q and O of its 32 rows for its half only (D/8 + D/4
// registers, at most 384), and per key tile
//   1. computes the partial S^T = K_half Q_half^T (32 keys x 32 queries);
//   2. swaps it with the wave holding the other half of the same rows through
//      LDS and adds (a + b is the same in either order, so both waves hold
//      identical scores and take identical softmax decisions);
//   3. runs the online softmax: a reference max per row, raised (with O
//      and l rescaled) only when a tile's max breaks it by more than tau;
//   4. accumulates O^T_half += V_half^T P^T.
// Tiles are 32 keys. A staged K tile holds both halves, each as 32 dense rows
// of W / 8 granules (dense_pos: granules swizzled inside groups of 16, 8 or
// 4 by the row, so that sixteen lanes reading sixteen rows hit distinct
// banks whatever the pitch), at most 64 KiB. Dense rows let every copy
// instruction carry a full 1 KiB: the copy path costs per instruction, not
// per byte. V is staged from its transposed copy (fwd_vt.hpp), written in
// blocks of 32 keys so that a tile is one contiguous block of D rows of 64
// bytes (64 KiB at D = 1024): every copy instruction then covers whole
// 128-byte lines, where rows of all positions gave 64-byte pieces D rows
// apart (8 % faster at D = 1024). The tile is read with plain 16-byte
// reads. As in the prefill kernel the copy of V(j) is issued when the K(j)
// phase starts and the copy of K(j+1) when the V(j) phase starts.
//
// What bounds it is the feed from L2: each staged byte serves 64 query rows
// (the fp32 O of more rows does not fit the register file at D = 1024), so
// a launch moves twice the prefill kernel's L2-to-LDS bytes per flop, at
// about the same aggregate rate (8.5-10 TB/s). Overlapping the softmax and the score
// swap with the MFMAs (a one-tile software pipeline) measured no faster.
//
// Accumulation is fp32 (the fp16-accumulator request maps to this kernel too:
// it is at least as accurate).
#pragma once

#include "ffpa_common.hpp"
#include "fwd_prefill.hpp"

namespace ffpa {

constexpr int kWideBc = 32;                      // keys per tile
constexpr int kWideTile = 64 * 1024;             // LDS buffer of one staged K or V^T tile

constexpr int kWideXchg = 4096;                  // per wave: a 32 x 32 fp32 tile
constexpr int kWideLds = 2 * kWideTile + 4 * kWideXchg;

template <int D, bool BF16, bool DROP = false>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fwd_wide_kernel(FwdArgs a) {
  static_assert(D % 64 == 0 && D > 512 && D <= 1024, "D must be a multiple of 64 in (512, 1024]");
  using E = Elem<BF16>;
  using V8 = typename E::vec8;
  constexpr int W = D / 2;              // elements per half
  constexpr int SG = W / 8;             // granules per half row (36 .. 64)
  constexpr int HALF = kWideBc * SG * 16;  // bytes of one dense K half-tile
  constexpr int NS = W / 16;            // k-steps of the partial product
  constexpr int NDB = W / 32;           // output d-blocks of the half
  constexpr int KB = 0, VB = kWideTile, XB = 2 * kWideTile;
  constexpr int kKAhead = 8;
  constexpr int kVAhead = 12;
  // fp32 accumulator d-blocks in AGPRs (beside the W/4 Q registers); the rest in VGPRs
  constexpr int kOAgpr = (256 - W / 4) / 16 < NDB ? (256 - W / 4) / 16 : NDB;

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = wave >> 1, hf = wave & 1;

  // ---- workgroup -> (b, h, block of 64 rows)
  const int n_qb = (a.Nq + 63) / 64;
  const int t = xcd_logical(blockIdx.x, a.total_wg);
  // causal: longest rows (last query blocks) first
  const int qb = a.causal ? n_qb - 1 - causal_position(t, n_qb, a.total_wg) : t % n_qb;
  const int bh = t / n_qb;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int q0 = qb * 64;
  const int qw = q0 + 32 * rb;        // first row of this wave

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * a.Nkv) * D * 2;
  const uint32_t kv_bytes = (uint32_t)a.Nkv * D * 2;  // rows >= Nkv read as zeros
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc((const char*)a.k + kv_off, kv_bytes);
  // V^T in blocks of one tile: [tile][d][32 keys], D * 64 bytes per tile
  constexpr uint32_t vt_row = kWideBc * 2;  // bytes per d row of a block
  const __amdgpu_buffer_rsrc_t Vr =
      make_rsrc((const char*)a.vt + (size_t)(b * a.Hkv + hk) * D * a.nkv_pad * 2, (uint32_t)D * a.nkv_pad * 2);

  int kv_end = a.Nkv;
  if (a.causal) kv_end = min(kv_end, min(q0 + 64, a.Nq));  // keys <= last row of the block
  const int n_tiles = (kv_end + kWideBc - 1) / kWideBc;
  const bool has_mask = a.mask_rows > 0;
  const uint16_t* mk = (const uint16_t*)a.mask;

  // ---- Q^T half in registers: lane holds Q[qw + l % 32][W hf + 16 s + 8 (l / 32) .. +7]
  u32x4 qf[NS];
  {
    const typename E::scalar* Q = (const typename E::scalar*)a.q + ((size_t)(b * a.Hq + h) * a.Nq) * D;
    const int qrow = min(qw + (lane & 31), a.Nq - 1);
    const u32x4* qp = (const u32x4*)(Q + (size_t)qrow * D + W * hf + 8 * (lane >> 5));
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = qp[2 * s];
  }
  // compiler-visible: without it the K-phase MFMAs of every tile would wait
  // for the Q loads again, and those waits also hold for the copies in flight
  wait_vmcnt0_visible();

  // ---- copies: instruction n of a tile (n = wave + 4 r, r < 16) fills half
  // n / 32 of key row n % 32; lane i writes slot i = logical granule i ^ swz4(row)
  // copy instruction n (n = wave + 4 r, r < SG / 4) fills 1 KiB of a dense
  // half-tile: half n / (SG / 2), slots 64 (n % (SG / 2)) + lane, slot s
  // holding granule dense_pos(row, s % SG) of row s / SG
  auto k_copy = [&](int tile, int r, int ln) {
    const int n = wave + 4 * r;
    const int half = n / (SG / 2), nn = n % (SG / 2);
    const int sl = 64 * nn + ln;
    const int row = sl / SG, g = dense_pos(SG, row, sl % SG);
    const uint32_t voff = (uint32_t)((half * W + 8 * g) * 2) + (uint32_t)(tile * kWideBc + row) * (D * 2);
    dma16(Kr, voff, smem + KB + half * HALF + nn * 1024);
  };
  auto issue_k_tile = [&](int tile) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int r = 0; r < SG / 4; ++r) k_copy(tile, r, ln);
  };

  // ---- copy of one V^T tile (D rows of 32 keys = 64 bytes). Copy
  // instruction n (n = wave + 4 r, r < D / 64) fills LDS rows 16 n .. 16 n +
  // 15: lane i writes slot i % 4 of row 16 n + i / 4, which holds the logical
  // granule (positions 8 g .. 8 g + 7) g = (i % 4) ^ ((row / 4) % 4), and
  // (row / 4) % 4 = (i / 16) % 4 whatever n is.
  auto vt_lane_offset = [&](int ln) {
    return (uint32_t)(ln >> 2) * vt_row + (uint32_t)(((ln & 3) ^ ((ln >> 4) & 3)) << 4);
  };
  auto vt_copy = [&](int tile, int r, uint32_t lo) {
    const int n = wave + 4 * r;
    dma16(Vr, lo + (uint32_t)(16 * n) * vt_row + (uint32_t)tile * (D * vt_row), smem + VB + n * 1024);
  };
  // The copies of a tile are spread over the first `span` MFMA steps of the
  // phase before the one that reads them (copy r at step r span / count):
  // issued in one burst, they held the wave's MFMAs back while the copy
  // instructions queued.
  constexpr int NKC = SG / 4, NVC = D / 64;  // copies per wave per tile: K, V^T
  // each phase issues the other buffer's copies over the first half of its
  // steps; above D = 768 over three quarters (1.4 % faster at D = 1024, no
  // faster at 576 and 768)
  constexpr int SPAN_NUM = D > 768 ? 3 : 2, SPAN_DEN = 4;

  // K fragment (A of S^T) for k-step st = 8 a + c: key row l % 32, granule 2 st + l / 32
  auto k_bases = [&](int ln, uint32_t* kx) {
    const int r = ln & 31, hh = ln >> 5;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      kx[c] = (uint32_t)(KB + hf * HALF + r * (SG * 16) + (dense_pos(SG, r, 2 * c + hh) << 4));
  };
  // V^T fragment (A of O^T_half) for d-block db and the 16-key step t2: row
  // W hf + 32 db + l % 32 of the V^T tile, logical granule 2 t2 + l / 32,
  // whose positions hold the keys the lane's P operand pairs with (vt_key).
  // Sixteen consecutive lanes read sixteen consecutive 64-byte rows: four
  // share a bank window, and (row / 4) % 4 spreads them over it.
  auto v_bases = [&](int ln, uint32_t* vx) {
    const int r = ln & 31, h = ln >> 5;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      vx[t2] = (uint32_t)(VB + (W * hf + r) * 64 + (((2 * t2 + h) ^ ((r >> 2) & 3)) << 4));
  };

  f32x16 o_acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o_acc[i] = f32x16{};
  float m_ref = -INFINITY;  // reference max (log2 domain)
  float l_run = 0.f;        // this lane's partial row sum
  bool fresh = true;        // no PV product accumulated yet

  if (n_tiles > 0) issue_k_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    const int j0 = j * kWideBc;
    int lj = lane;
    asm volatile("" : "+v"(lj));
    const int hij = lj >> 5;
    const int my_qj = qw + (lj & 31);
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      if (d < kOAgpr) asm volatile("" : "+a"(o_acc[d]));
      else asm volatile("" : "+v"(o_acc[d]));
    }
    // dropout keep bit i of the lane's row against key j0 + 4 hi + 8 (i / 4)
    // + i % 4 (the quad's four generator calls, one a lane), made before the
    // products while fewer registers are live
    const uint32_t keep = DROP ? drop_bits_row(a.drop, b * a.Hq + h, my_qj, j0 + 4 * hij) : 0u;

    // ===== K phase: partial S^T over this half, two chains (even / odd k-steps)
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    f32x16 s_acc, s_odd;
    {
      uint32_t vlo;
      {
        int lnc = lane;
        asm volatile("" : "+v"(lnc));
        vlo = vt_lane_offset(lnc);
        asm volatile("" : "+v"(vlo));  // opaque: each copy then adds a scalar offset
      }
      u32x4 kf[kKAhead];
      uint32_t kx[8];
      k_bases(lj, kx);
      auto kread = [&](int st) { return lds_read16(smem + kx[st & 7] + 256 * (st >> 3)); };
#pragma unroll
      for (int st = 0; st < kKAhead; ++st) kf[st] = kread(st);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
#pragma unroll
        for (int r = 0; r < NVC; ++r)
          if ((r * (SPAN_NUM * NS / SPAN_DEN)) / NVC == st) vt_copy(j, r, vlo);
        const u32x4 a0 = kf[st % kKAhead];
        if (st + kKAhead < NS) kf[st % kKAhead] = kread(st + kKAhead);
        f32x16& acc = (st & 1) ? s_odd : s_acc;
        if (st < 2) mfma32_asm<BF16, true, false, true>(acc, a0, qf[st]);
        else if (st == NS - 1) mfma32_asm<BF16, true, false, false, false, true>(acc, a0, qf[st]);
        else mfma32_asm<BF16, true, false>(acc, a0, qf[st]);
      }
    }
    // both chains end at least 19 wait states before this VALU (the last MFMA pads)
    pin_after_pad(s_acc);
    pin_after_pad(s_odd);
#pragma unroll
    for (int i = 0; i < 16; ++i) s_acc[i] += s_odd[i];

    // ===== swap partial scores with the other half's wave; add
    {
      FFPA_LDS f32x4* mine = (FFPA_LDS f32x4*)(smem + XB + wave * kWideXchg) + lj;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        mine[64 * jj] = f32x4{s_acc[4 * jj], s_acc[4 * jj + 1], s_acc[4 * jj + 2], s_acc[4 * jj + 3]};
      wait_lgkm0();
      barrier();
      const FFPA_LDS f32x4* other = (const FFPA_LDS f32x4*)(smem + XB + (wave ^ 1) * kWideXchg) + lj;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 x = other[64 * jj];
#pragma unroll
        for (int e = 0; e < 4; ++e) s_acc[4 * jj + e] += x[e];
      }
    }

    // ===== online softmax (log2 domain); register i holds key j0 + 8 (i/4) + 4 hi + i%4
    const int kb0 = j0 + 4 * hij;
    const bool need_mask = has_mask || (j0 + kWideBc > a.Nkv) || (a.causal && j0 + kWideBc - 1 > qw);
    float tv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) tv[i] = s_acc[i] * a.scale_log2;
    if (need_mask) {
      // key bias, or row my_q of a per-query mask (clamped to the last row)
      const uint16_t* mrow = mk + (size_t)min(my_qj, a.Nq - 1) * a.mask_stride;
      int klim = a.Nkv - kb0;
      if (a.causal) klim = min(klim, my_qj + 1 - kb0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = 8 * (i >> 2) + (i & 3);
        if (has_mask) tv[i] += E::to_f32(mrow[min(kb0 + c, a.Nkv - 1)]) * kLog2e;
        tv[i] = c >= klim ? -INFINITY : tv[i];
      }
    }
    float mx = tv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, tv[i]);
    mx = fmaxf(mx, swap_halves(mx));
    // The reference max rises (and O and l follow it) when a row's max breaks
    // m_ref + tau; P = 2^(t - m_ref) then stays within 2^tau. The two waves
    // of a pair hold identical scores, so they take identical decisions.
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + fwd_tau<BF16>()) != 0) {  // wave-uniform
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
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
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      tv[i] = exp2_fast(tv[i] - m_use);
      psum += tv[i];
    }
    l_run += psum;
    if constexpr (DROP) {
      // dropout: the row sum keeps the undropped P, O gets the scale of the
      // kept elements at the end
#pragma unroll
      for (int i = 0; i < 16; ++i) tv[i] = keep_if_bit(tv[i], keep, i);
    }
    V8 pf[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const float* x = &tv[8 * t2];
      pf[t2] = pack8<BF16>(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(pf[t2]));

    // ===== V phase: O^T_half += V_half^T P^T
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    // The PV products, as a lambda instantiated for the first tile of an
    // attempt (FRESH: the t2 = 0 product of each block starts from C = 0) and
    // for the others, so that no MFMA of the hot loop sits behind a branch.
    auto v_phase = [&](auto fresh_tag) {
      constexpr bool FRESH = decltype(fresh_tag)::value;
      constexpr int NSV = 2 * NDB;  // steps st = NDB t2 + db
      uint32_t vx[2];
      {
        int lv = lane;
        asm volatile("" : "+v"(lv));
        v_bases(lv, vx);
      }
      auto vread = [&](int st) {
        const int db = st % NDB, t2 = st / NDB;
        return lds_read16(smem + vx[t2] + 2048 * db);
      };
      u32x4 vf[kVAhead];
#pragma unroll
      for (int st = 0; st < kVAhead; ++st) vf[st] = vread(st);
      int lnc = lane;
      asm volatile("" : "+v"(lnc));
#pragma unroll
      for (int st = 0; st < NSV; ++st) {
        // K(j+1); on the last tile rows past the key range (range-checked
        // zeros) or, causal, rows nobody reads: harmless, and branch-free
#pragma unroll
        for (int r = 0; r < NKC; ++r)
          if ((r * (SPAN_NUM * NSV / SPAN_DEN)) / NKC == st) k_copy(j + 1, r, lnc);
        const int db = st % NDB, t2 = st / NDB;
        const u32x4 vbits = vf[st % kVAhead];
        if (st + kVAhead < NSV) vf[st % kVAhead] = vread(st + kVAhead);
        const u32x4 pb = __builtin_bit_cast(u32x4, pf[t2]);
        // the first MFMA pads for the VALU that wrote P, the last one for
        // whatever the compiler places after the phase on any path
        const bool zero = FRESH && t2 == 0;
        const bool pad_after = st == NSV - 1;
        if (db < kOAgpr) {
          if (zero) {
            if (st == 0) mfma32_asm<BF16, false, true, true, true>(o_acc[db], vbits, pb);
            else mfma32_asm<BF16, false, true, true>(o_acc[db], vbits, pb);
          } else if (st == 0) {
            mfma32_asm<BF16, false, true, false, true>(o_acc[db], vbits, pb);
          } else if (pad_after) {
            mfma32_asm<BF16, false, true, false, false, true>(o_acc[db], vbits, pb);
          } else {
            mfma32_asm<BF16, false, true>(o_acc[db], vbits, pb);
          }
        } else {
          if (zero) {
            if (st == 0) mfma32_asm<BF16, false, false, true, true>(o_acc[db], vbits, pb);
            else mfma32_asm<BF16, false, false, true>(o_acc[db], vbits, pb);
          } else if (st == 0) {
            mfma32_asm<BF16, false, false, false, true>(o_acc[db], vbits, pb);
          } else if (pad_after) {
            mfma32_asm<BF16, false, false, false, false, true>(o_acc[db], vbits, pb);
          } else {
            mfma32_asm<BF16, false, false>(o_acc[db], vbits, pb);
          }
        }
      }
    };
    if (fresh) v_phase(BoolTag<true>{});
    else v_phase(BoolTag<false>{});
    fresh = false;
  }
  wait_vmcnt<0>();
  asm volatile("s_nop 7\n s_nop 7\n s_nop 4" ::: "memory");
#pragma unroll
  for (int d = 0; d < NDB; ++d) {
    if (d < kOAgpr) asm volatile("" : "+a"(o_acc[d]));
    else asm volatile("" : "+v"(o_acc[d]));
  }

  // ===== epilogue: rows of the half through LDS (32 rows x 1 KiB per wave),
  // then stored as contiguous pieces of W elements per row
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * (DROP ? a.drop.scale : 1.f);
  wait_lgkm0();
  barrier();
  FFPA_LDS char* ostage = smem + wave * 32 * 1024;
  {
    const int r = lane & 31, hie = lane >> 5;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 st = {E::pack2(o_acc[db][4 * g4] * inv, o_acc[db][4 * g4 + 1] * inv),
                          E::pack2(o_acc[db][4 * g4 + 2] * inv, o_acc[db][4 * g4 + 3] * inv)};
        const int g = 4 * db + g4;
        *(FFPA_LDS u32x2*)(ostage + r * 1024 + ((g ^ (r & 15)) << 4) + 8 * hie) = st;
      }
  }
  {
    typename E::scalar* O = (typename E::scalar*)a.o + ((size_t)(b * a.Hq + h) * a.Nq + qw) * D + W * hf;
    const int rows = min(32, a.Nq - qw);
    constexpr int NIT = (32 * SG + 63) / 64;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = it * 64 + lane;
      const int r = c / SG, g = c % SG;
      if (r < rows) {
        const u32x4 x = *(const FFPA_LDS u32x4*)(ostage + r * 1024 + ((g ^ (r & 15)) << 4));
        *(u32x4*)(O + (size_t)r * D + 8 * g) = x;
      }
    }
  }
  if (hf == 0 && a.lse != nullptr && (lane >> 5) == 0 && qw + lane < a.Nq) {
    float* L = a.lse + (size_t)(b * a.Hq + h) * a.Nq + qw + lane;
    *L = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

// Host launcher: the transposed copy of V (blocks of 32 keys) into a.vt, then
// the kernel. The LDS limit is set before anything is enqueued.
template <int D, bool BF16, bool DROP = false>
hipError_t launch_fwd_wide(const FwdArgs& a, hipStream_t stream) {
  auto kern = fwd_wide_kernel<D, BF16, DROP>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kWideLds);
  if (attr != hipSuccess) return attr;
  const hipError_t e = launch_fwd_vt(a.v, const_cast<void*>(a.vt), a.B * a.Hkv, a.Nkv, D, kWideBc, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.total_wg), dim3(256), kWideLds, stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
