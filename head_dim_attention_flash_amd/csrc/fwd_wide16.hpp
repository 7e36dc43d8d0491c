// Forward attention above D = 512 with the output accumulator held in fp16
// (the "ACC+F16" variant of "FFPA-Attn Performance Benchmarks on Lambda.ai",
// sections 1-3, and "Why the Trends Look Like This", F16 vs F32
// accumulation). Same operation as fwd_wide.hpp: O = softmax(scale Q K^T +
// mask) V and lse per row ("naive_math", section 3 of the
// attention-kernel-profiler design document), masks and GQA as there.
//
// gfx950 has no MFMA with an fp16 result: scores and each tile's P V products
// are fp32 MFMA accumulators; the running O is packed fp16, kept normalised
// (O <- O * (alpha l_old / l_new) + (P / l_new) V, one packed fp16 FMA per
// pair of elements per tile), so |O| never exceeds max |V|.
//
// Why a kernel of its own: the fp16 O takes half the registers of the fp32
// one. Up to D = 768 a wave then holds Q and O of its 32 rows for all of D
// (D / 4 + D / 4 registers), like the prefill kernel does up to D = 512 with
// an fp32 O, and a workgroup serves 128 rows: per staged K and V^T byte twice
// the rows of the fp32 wide kernel (what bounds that one is the feed of
// staged bytes from L2), no partial scores to swap between waves, and one
// softmax per row. Above D = 768 Q and O of 32 rows exceed a wave's
// registers, and D is split across wave pairs as in fwd_wide.hpp (64 rows
// per workgroup; per tile the pair swaps its partial S^T through LDS and
// adds, a + b being the same in either order, so both waves take identical
// softmax decisions).
//
// Per 32-key tile each wave computes S^T over its part of D (two MFMA chains,
// even and odd k-steps), [swaps and adds,] rescales, and accumulates
// O^T += V^T P^T into per-tile fp32 products of two d-blocks at a time, folded
// into the fp16 O while the next two d-blocks' products run. Staging as in
// fwd_wide.hpp: a K tile of 32 keys as dense rows (one part-tile per part of
// D), a V^T tile of D rows of 32 keys from the transposed copy in blocks of
// 32 keys; the copies of V(j) are spread over the K(j) phase and those of
// K(j + 1) over the V(j) phase.
#pragma once

#include "ffpa_common.hpp"
#include "fwd_prefill.hpp"
#include "fwd_wide.hpp"

namespace ffpa {

// parts of D per row block: 1 (a wave holds all of D for its rows) or 2 (a
// wave pair splits D). The default: 1 up to D = 768 (above, all of D does not
// fit a wave's registers); 2 is built for every D as the other tile shape.
template <int D>
constexpr int wide16_nh() {
  return D <= 768 ? 1 : 2;
}
// query rows per workgroup: 4 / NH row blocks of 32
template <int D, int NH = wide16_nh<D>()>
constexpr int wide16_rows() {
  return (4 / NH) * 32;
}
// LDS bytes of one staged K or V^T tile (32 keys x D)
template <int D>
constexpr int wide16_tile() {
  return kWideBc * D * 2;
}
// The epilogue stages each wave's 32 rows x W columns (W = D / NH) through
// LDS in one pass, or two passes of W / 2 columns when W > 512; a staged row
// takes whole groups of 16 granules.
template <int D, int NH = wide16_nh<D>()>
constexpr int wide16_epi_passes() {
  return D / NH > 512 ? 2 : 1;
}
template <int D, int NH = wide16_nh<D>()>
constexpr int wide16_pitch() {
  return (D / NH / wide16_epi_passes<D, NH>() / 8 + 15) / 16 * 256;
}
// LDS: two tiles and, NH = 2, the score swap area; or the epilogue's staging
// if that is larger
template <int D, int NH = wide16_nh<D>()>
constexpr int wide16_lds() {
  constexpr int loop = 2 * wide16_tile<D>() + (NH == 2 ? 4 * kWideXchg : 0);
  constexpr int epi = 4 * 32 * wide16_pitch<D, NH>();
  return loop > epi ? loop : epi;
}

template <int D, bool BF16, int NH = wide16_nh<D>()>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fwd_wide16_kernel(FwdArgs a) {
  static_assert(D % 64 == 0 && D > 512 && D <= 1024, "D must be a multiple of 64 in (512, 1024]");
  static_assert(NH == 2 || D <= 768, "a wave holds all of D only up to D = 768");
  using E = Elem<BF16>;
  using V8 = typename E::vec8;
  constexpr int ROWS = wide16_rows<D, NH>();
  constexpr int W = D / NH;                // elements per part of D
  constexpr int SG = W / 8;                // granules per part of a row (36 .. 96)
  constexpr int PART = kWideBc * SG * 16;  // bytes of one dense K part-tile
  constexpr int NS = W / 16;               // k-steps of the (partial) product
  constexpr int NDB = W / 32;              // output d-blocks of the part
  constexpr int TILE = wide16_tile<D>();
  constexpr int KB = 0, VB = TILE, XB = 2 * TILE;
  constexpr int kKAhead = 8;               // K fragments read ahead
  constexpr int kVAhead = 4;               // V^T fragments read ahead
  constexpr int NKC = D / 64, NVC = D / 64;  // copy instructions per wave per tile: K, V^T
  // P V products go in groups of two d-blocks (the last group alone when NDB
  // is odd); a group's MFMAs run (d0, t2 0), (d1, t2 0), (d0, t2 1), (d1, t2 1),
  // so that consecutive MFMAs write different accumulators
  constexpr int NSV = 2 * NDB;  // MFMA steps of the V phase
  // each phase issues the other buffer's copies over its first half of MFMA
  // steps (NH = 2: three quarters, 3 % faster at D = 1024; NH = 1 is no
  // faster that way, and D = 768 then spills)
  constexpr int KSPAN = NH == 2 ? 3 * NS / 4 : NS / 2;
  constexpr int VSPAN = NH == 2 ? 3 * NSV / 4 : NSV / 2;
  static_assert(NS % 2 == 0, "two score chains of equal length");

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave / NH, hf = wave % NH;  // row block, part of D

  // ---- workgroup -> (b, h, block of ROWS rows)
  const int n_qb = (a.Nq + ROWS - 1) / ROWS;
  const int t = xcd_logical(blockIdx.x, a.total_wg);
  // causal: longest rows (last query blocks) first
  const int qb = a.causal ? n_qb - 1 - causal_position(t, n_qb, a.total_wg) : t % n_qb;
  const int bh = t / n_qb;
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int q0 = qb * ROWS;
  const int qw = q0 + 32 * rg;  // first row of this wave

  const size_t kv_off = ((size_t)(b * a.Hkv + hk) * a.Nkv) * D * 2;
  const uint32_t kv_bytes = (uint32_t)a.Nkv * D * 2;  // rows >= Nkv read as zeros
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc((const char*)a.k + kv_off, kv_bytes);
  constexpr uint32_t vt_row = kWideBc * 2;  // bytes per d row of a V^T block
  const __amdgpu_buffer_rsrc_t Vr =
      make_rsrc((const char*)a.vt + (size_t)(b * a.Hkv + hk) * D * a.nkv_pad * 2, (uint32_t)D * a.nkv_pad * 2);

  int kv_end = a.Nkv;
  if (a.causal) kv_end = min(kv_end, min(q0 + ROWS, a.Nq));  // keys <= last row of the block
  const int n_tiles = (kv_end + kWideBc - 1) / kWideBc;
  const bool has_mask = a.mask_rows > 0;
  const uint16_t* mk = (const uint16_t*)a.mask;

  // ---- Q^T part in registers: lane holds Q[qw + l % 32][W hf + 16 s + 8 (l / 32) .. +7]
  u32x4 qf[NS];
  {
    const typename E::scalar* Q = (const typename E::scalar*)a.q + ((size_t)(b * a.Hq + h) * a.Nq) * D;
    const int qrow = min(qw + (lane & 31), a.Nq - 1);
    const u32x4* qp = (const u32x4*)(Q + (size_t)qrow * D + W * hf + 8 * (lane >> 5));
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = qp[2 * s];
  }
  // compiler-visible: later waits then never hold for the copies in flight
  wait_vmcnt0_visible();

  // ---- copies (the layouts of fwd_wide.hpp). K instruction n (n = wave + 4 r,
  // r < D / 64) fills 1 KiB of a dense part-tile: part n / (SG / 2), slots
  // 64 (n % (SG / 2)) + lane, slot s holding granule dense_pos(row, s % SG) of
  // row s / SG. V^T instruction n (r < D / 64) fills V^T rows 16 n .. 16 n + 15.
  // The lane's offset within a tile for each of its K copies is computed once
  // (a division by the row pitch and the swizzle: ~15 VALU instructions per
  // copy and tile otherwise) and kept in spare AGPRs; a copy then costs a
  // register read and the tile's offset.
  uint32_t koff[NKC];
#pragma unroll
  for (int r = 0; r < NKC; ++r) {
    const int n = wave + 4 * r;
    const int part = n / (SG / 2), nn = n % (SG / 2);
    const int sl = 64 * nn + lane;
    const int row = sl / SG, g = dense_pos(SG, row, sl % SG);
    koff[r] = (uint32_t)((part * W + 8 * g) * 2) + (uint32_t)row * (D * 2);
  }
  auto k_copy = [&](int tile, int r) {
    const int n = wave + 4 * r;
    const int part = n / (SG / 2), nn = n % (SG / 2);
    dma16(Kr, koff[r] + (uint32_t)(tile * kWideBc) * (D * 2), smem + KB + part * PART + nn * 1024);
  };
  auto issue_k_tile = [&](int tile) {
#pragma unroll
    for (int r = 0; r < NKC; ++r) k_copy(tile, r);
  };
  auto vt_lane_offset = [&](int ln) {
    return (uint32_t)(ln >> 2) * vt_row + (uint32_t)(((ln & 3) ^ ((ln >> 4) & 3)) << 4);
  };
  auto vt_copy = [&](int tile, int r, uint32_t lo) {
    const int n = wave + 4 * r;
    dma16(Vr, lo + (uint32_t)(16 * n) * vt_row + (uint32_t)tile * (D * vt_row), smem + VB + n * 1024);
  };
  // K fragment (A of S^T) for k-step st = 8 a + c: key row l % 32, granule 2 st + l / 32
  auto k_bases = [&](int ln, uint32_t* kx) {
    const int r = ln & 31, hh = ln >> 5;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      kx[c] = (uint32_t)(KB + hf * PART + r * (SG * 16) + (dense_pos(SG, r, 2 * c + hh) << 4));
  };
  // V^T fragment (A of O^T) for d-block db and 16-key step t2: row
  // W hf + 32 db + l % 32 of the tile, logical granule 2 t2 + l / 32 (vt_key order)
  auto v_bases = [&](int ln, uint32_t* vx) {
    const int r = ln & 31, hh = ln >> 5;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      vx[t2] = (uint32_t)(VB + (W * hf + r) * 64 + (((2 * t2 + hh) ^ ((r >> 2) & 3)) << 4));
  };

  // ---- fp16 output accumulator: block db holds O^T[32 db .. +31][row] of the
  // lane's row as 16 packed fp16 (two u32x4: elements 0-7, 8-15 of the MFMA C
  // layout)
  u32x4 o16[NDB][2];
#pragma unroll
  for (int d = 0; d < NDB; ++d) o16[d][0] = o16[d][1] = u32x4{0, 0, 0, 0};
  float m_ref = -INFINITY;  // reference max (log2 domain)
  float l_run = 0.f;        // the full row sum, relative to m_ref

  if (n_tiles > 0) issue_k_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    const int j0 = j * kWideBc;
#pragma unroll
    for (int r = 0; r < NKC; ++r) asm volatile("" : "+a"(koff[r]));
    int lj = lane;
    asm volatile("" : "+v"(lj));
    const int hij = lj >> 5;
    const int my_q = qw + (lj & 31);

    // ===== K phase: S^T (NH = 2: partial, over this part of D)
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    f32x16 s_acc, s_odd;  // two chains: even / odd k-steps
    {
      uint32_t vlo;
      {
        int lnc = lane;
        asm volatile("" : "+v"(lnc));
        vlo = vt_lane_offset(lnc);
        asm volatile("" : "+v"(vlo));
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
          if ((r * KSPAN) / NVC == st) vt_copy(j, r, vlo);
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

    // ===== NH = 2: swap partial scores with the other part's wave; add
    if constexpr (NH == 2) {
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

    // ===== online softmax (log2 domain), renormalised every tile; register i
    // of the scores holds key j0 + 8 (i / 4) + 4 hi + i % 4
    V8 pf[2];
    float oscale;
    {
      const int kb0 = j0 + 4 * hij;
      const bool need_mask = has_mask || (j0 + kWideBc > a.Nkv) || (a.causal && j0 + kWideBc - 1 > qw);
      float tv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tv[i] = s_acc[i] * a.scale_log2;
      if (need_mask) {
        const uint16_t* mrow = mk + (size_t)min(my_q, a.Nq - 1) * a.mask_stride;
        int klim = a.Nkv - kb0;
        if (a.causal) klim = min(klim, my_q + 1 - kb0);
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
      float alpha = 1.f;
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleTau) != 0) {  // wave-uniform
        const float m_new = fmaxf(m_ref, mx);
        alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_ref - m_new);
        m_ref = m_new;
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        tv[i] = exp2_fast(tv[i] - m_use);
        psum += tv[i];
      }
      const float l_old = l_run;
      const float l_new = alpha * l_old + psum + swap_halves(psum);
      l_run = l_new;
      const float pscale = l_new > 0.f ? 1.f / l_new : 0.f;
      oscale = alpha * l_old * pscale;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const float* x = &tv[8 * t2];
        pf[t2] = pack8<BF16>(x[0] * pscale, x[1] * pscale, x[2] * pscale, x[3] * pscale, x[4] * pscale,
                             x[5] * pscale, x[6] * pscale, x[7] * pscale);
      }
    }
    // P is the B operand of inline-asm MFMAs: every VALU write of it happens
    // here, before the barrier (the first MFMA of the phase pads as well)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(pf[t2]));

    // ===== V phase: per-tile products V^T P^T, folded into the fp16 O
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    {
      uint32_t vx[2];
      {
        int lv = lane;
        asm volatile("" : "+v"(lv));
        v_bases(lv, vx);
      }
      // step s -> group g = s / 4, d-block of the group uu, key step t2
      auto step_of = [](int s, int& g, int& uu, int& t2) {
        g = s >> 2;
        const int k = s & 3;
        const bool pair = 2 * g + 1 < NDB;
        uu = pair ? (k & 1) : 0;
        t2 = pair ? (k >> 1) : k;
      };
      auto vread = [&](int s) {
        int g, uu, t2;
        step_of(s, g, uu, t2);
        return lds_read16(smem + vx[t2] + 2048 * (2 * g + uu));
      };
      u32x4 vf[kVAhead];
#pragma unroll
      for (int s = 0; s < kVAhead && s < NSV; ++s) vf[s] = vread(s);

      f32x16 pv[2][2];  // [set = group % 2][d-block of the group]
      const f16x2 sc = {(_Float16)oscale, (_Float16)oscale};
      // o16 <- o16 * oscale + acc, in packed fp16
      auto fold_block = [&](const f32x16& acc, int db) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 w = o16[db][hh];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f16x2 cur = f16x2_from_bits(w[e]);
            const f16x2 add = {(_Float16)acc[8 * hh + 2 * e], (_Float16)acc[8 * hh + 2 * e + 1]};
            cur = cur * sc + add;
            w[e] = __builtin_bit_cast(uint32_t, cur);
          }
          o16[db][hh] = w;
        }
      };
      // A group's fold runs as one block of VALU work between the MFMAs of
      // the next two groups: spread in quarters between the next group's
      // MFMAs it measured 8-9 % slower.
      auto fold_group = [&](int g) {
        fold_block(pv[g & 1][0], 2 * g);
        if (2 * g + 1 < NDB) fold_block(pv[g & 1][1], 2 * g + 1);
        // the folded values exist here, before the next MFMAs (which reuse
        // this set's registers two groups later)
        asm volatile("" : "+v"(o16[2 * g][0]), "+v"(o16[2 * g][1]));
        if (2 * g + 1 < NDB) asm volatile("" : "+v"(o16[2 * g + 1][0]), "+v"(o16[2 * g + 1][1]));
      };
#pragma unroll
      for (int s = 0; s < NSV; ++s) {
        // K(j+1); on the last tile rows past the key range (range-checked
        // zeros) or, causal, rows nobody reads: harmless, and branch-free
#pragma unroll
        for (int r = 0; r < NKC; ++r)
          if ((r * VSPAN) / NKC == s) k_copy(j + 1, r);
        int g, uu, t2;
        step_of(s, g, uu, t2);
        const u32x4 vbits = vf[s % kVAhead];
        if (s + kVAhead < NSV) vf[s % kVAhead] = vread(s + kVAhead);
        const u32x4 pb = __builtin_bit_cast(u32x4, pf[t2]);
        f32x16& acc = pv[g & 1][uu];
        // padded after: the last step (the last group folds right after it)
        // and the last step of group 1, before group 0's fold, which no
        // earlier fold separates from group 0's MFMAs
        const bool pad = s == NSV - 1 || s == 7;
        if (t2 == 0) {
          if (s == 0) mfma32_asm<BF16, false, false, true, true>(acc, vbits, pb);
          else mfma32_asm<BF16, false, false, true>(acc, vbits, pb);
        } else if (pad) {
          mfma32_asm<BF16, false, false, false, false, true>(acc, vbits, pb);
        } else {
          mfma32_asm<BF16, false, false>(acc, vbits, pb);
        }
        // group g - 1 folds once group g's MFMAs have issued; its products are
        // pinned after them so the fold cannot move up next to its own MFMAs
        const bool group_end = (s & 3) == 3 || s == NSV - 1;
        if (group_end && g > 0) {
          pin_after_pad(pv[(g - 1) & 1][0]);
          pin_after_pad(pv[(g - 1) & 1][1]);
          fold_group(g - 1);
        }
        if (s == NSV - 1) {
          // the last MFMA padded: the last group folds now
          pin_after_pad(pv[g & 1][0]);
          pin_after_pad(pv[g & 1][1]);
          fold_group(g);
        }
      }
    }
  }
  wait_vmcnt<0>();  // no copy may still target this workgroup's LDS when it ends

  // ===== epilogue: the wave's 32 rows of its part go through LDS (in EP
  // passes of W / EP columns, a staged row taking whole groups of 16
  // granules), then out as contiguous pieces of W / EP elements per row
  constexpr int EP = wide16_epi_passes<D, NH>();
  constexpr int NDBP = NDB / EP;   // d-blocks per pass
  constexpr int SGP = 4 * NDBP;    // granules per row and pass
  constexpr int PITCH = wide16_pitch<D, NH>();
  static_assert(NDB % EP == 0 && PITCH >= SGP * 16, "epilogue passes");
  static_assert(4 * 32 * PITCH <= wide16_lds<D, NH>(), "epilogue staging fits the LDS");
  wait_lgkm0();
  barrier();  // every wave is done with the tile buffers
  FFPA_LDS char* ostage = smem + wave * 32 * PITCH;
#pragma unroll
  for (int pe = 0; pe < EP; ++pe) {
    {
      const int rr = lane & 31, hie = lane >> 5;
#pragma unroll
      for (int dq = 0; dq < NDBP; ++dq)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x4 w = o16[NDBP * pe + dq][g4 >> 1];
          const f16x2 p0 = f16x2_from_bits(w[2 * (g4 & 1)]);
          const f16x2 p1 = f16x2_from_bits(w[2 * (g4 & 1) + 1]);
          const u32x2 st = {E::pack2((float)p0[0], (float)p0[1]), E::pack2((float)p1[0], (float)p1[1])};
          const int gg = 4 * dq + g4;  // elements 32 dq + 8 g4 + 4 hi .. +3 of the pass
          *(FFPA_LDS u32x2*)(ostage + rr * PITCH + ((gg ^ (rr & 15)) << 4) + 8 * hie) = st;
        }
    }
    {
      typename E::scalar* O =
          (typename E::scalar*)a.o + ((size_t)(b * a.Hq + h) * a.Nq + qw) * D + W * hf + 32 * NDBP * pe;
      const int rows = min(32, a.Nq - qw);
      constexpr int NIT = (32 * SGP + 63) / 64;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int c = it * 64 + lane;
        const int rr = c / SGP, gg = c % SGP;
        if (rr < rows) {
          const u32x4 x = *(const FFPA_LDS u32x4*)(ostage + rr * PITCH + ((gg ^ (rr & 15)) << 4));
          *(u32x4*)(O + (size_t)rr * D + 8 * gg) = x;
        }
      }
    }
  }
  if (hf == 0 && a.lse != nullptr && (lane >> 5) == 0 && qw + lane < a.Nq) {
    float* L = a.lse + (size_t)(b * a.Hq + h) * a.Nq + qw + lane;
    *L = l_run > 0.f ? (m_ref + __builtin_amdgcn_logf(l_run)) * kLn2 : -INFINITY;
  }
}

// Host launcher: the transposed copy of V (blocks of 32 keys) into a.vt, then
// the kernel over ceil(Nq / wide16_rows<D, NH>()) row blocks per head (the
// caller sets a.total_wg for that shape). The LDS limit is set before
// anything is enqueued.
template <int D, bool BF16, int NH = wide16_nh<D>()>
hipError_t launch_fwd_wide16(const FwdArgs& a, hipStream_t stream) {
  auto kern = fwd_wide16_kernel<D, BF16, NH>;
  constexpr int lds = wide16_lds<D, NH>();
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  const hipError_t e = launch_fwd_vt(a.v, const_cast<void*>(a.vt), a.B * a.Hkv, a.Nkv, D, kWideBc, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.total_wg), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
