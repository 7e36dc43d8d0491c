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
// one, and what bounds the wide forward is the feed of staged K and V^T
// bytes from L2 into each workgroup's LDS, which shrinks with the query rows
// a workgroup serves. Up to D = 768 a wave here holds two row blocks of 32
// queries (Q and O of 64 rows for its half of D: W / 2 + W / 2 registers,
// W = D / 2), so a workgroup serves 128 rows per staged byte, twice the fp32
// kernel's 64, and every K or V^T fragment read from LDS feeds two MFMAs.
// Above D = 768 two row blocks do not fit beside the per-tile products, and
// a wave holds one row block (64 rows per workgroup).
//
// Layout (as fwd_wide.hpp): 4 waves = 2 row groups x 2 halves of D; a K tile
// is 32 keys in two dense half-tiles, a V^T tile D rows of 32 keys from the
// transposed copy in blocks of 32 keys; per tile each wave computes the
// partial S^T over its half, swaps it with the wave holding the other half of
// the same rows through LDS and adds (a + b is the same in either order, so
// both waves take identical softmax decisions), rescales, and accumulates
// O^T_half += V_half^T P^T into per-tile fp32 products that are folded into
// the fp16 O while the next products run.
#pragma once

#include "ffpa_common.hpp"
#include "fwd_prefill.hpp"
#include "fwd_wide.hpp"

namespace ffpa {

// row blocks of 32 queries per wave
template <int D>
constexpr int wide16_rb() {
  return D <= 768 ? 2 : 1;
}
// query rows per workgroup
template <int D>
constexpr int wide16_rows() {
  return 64 * wide16_rb<D>();
}
// LDS bytes of one staged K or V^T tile (32 keys x D)
template <int D>
constexpr int wide16_tile() {
  return kWideBc * D * 2;
}
// bytes per row of the epilogue's staging: whole groups of 16 granules
template <int D>
constexpr int wide16_pitch() {
  return (D / 16 + 15) / 16 * 256;
}
// LDS: two tiles and the score swap area, or the epilogue's staging of 32
// rows per wave if that is larger
template <int D>
constexpr int wide16_lds() {
  constexpr int loop = 2 * wide16_tile<D>() + 4 * wide16_rb<D>() * kWideXchg;
  constexpr int epi = 4 * 32 * wide16_pitch<D>();
  return loop > epi ? loop : epi;
}

template <int D, bool BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void fwd_wide16_kernel(FwdArgs a) {
  static_assert(D % 64 == 0 && D > 512 && D <= 1024, "D must be a multiple of 64 in (512, 1024]");
  using E = Elem<BF16>;
  using V8 = typename E::vec8;
  constexpr int RB = wide16_rb<D>();
  constexpr int ROWS = wide16_rows<D>();
  constexpr int W = D / 2;                 // elements per half
  constexpr int SG = W / 8;                // granules per half row (36 .. 64)
  constexpr int HALF = kWideBc * SG * 16;  // bytes of one dense K half-tile
  constexpr int NS = W / 16;               // k-steps of the partial product
  constexpr int NDB = W / 32;              // output d-blocks of the half
  constexpr int TILE = wide16_tile<D>();
  constexpr int KB = 0, VB = TILE, XB = 2 * TILE;
  // fragments read ahead (registers are short with two row blocks)
  constexpr int kKAhead = RB == 2 ? (D > 640 ? 4 : 6) : 8;
  constexpr int kVAhead = RB == 2 && D > 704 ? 2 : 4;
  constexpr int NKC = SG / 4, NVC = D / 64;  // copy instructions per wave per tile: K, V^T
  // P V products: unit u = (d-block, row block); units go in groups of two
  // (the same d-block for both row blocks when RB = 2, two d-blocks when
  // RB = 1), each group's MFMAs in the order (u0, t2 0), (u1, t2 0), (u0, t2 1),
  // (u1, t2 1), so that consecutive MFMAs write different accumulators.
  constexpr int NU = NDB * RB;
  constexpr int NG = (NU + 1) / 2;
  constexpr int NSV = 2 * NU;  // MFMA steps of the V phase

  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  FFPA_LDS char* smem = (FFPA_LDS char*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave >> 1, hf = wave & 1;

  // ---- workgroup -> (b, h, block of ROWS rows)
  const int n_qb = (a.Nq + ROWS - 1) / ROWS;
  const int t = xcd_logical(blockIdx.x, a.total_wg);
  int qb = t % n_qb;
  const int bh = t / n_qb;
  if (a.causal) qb = n_qb - 1 - qb;  // longest rows first
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int q0 = qb * ROWS;
  const int qg = q0 + 32 * RB * rg;  // first row of this wave; block r starts at qg + 32 r

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

  // ---- Q^T halves in registers: lane holds Q[qg + 32 r + l % 32][W hf + 16 s + 8 (l / 32) .. +7]
  u32x4 qf[RB][NS];
  {
    const typename E::scalar* Q = (const typename E::scalar*)a.q + ((size_t)(b * a.Hq + h) * a.Nq) * D;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int qrow = min(qg + 32 * r + (lane & 31), a.Nq - 1);
      const u32x4* qp = (const u32x4*)(Q + (size_t)qrow * D + W * hf + 8 * (lane >> 5));
#pragma unroll
      for (int s = 0; s < NS; ++s) qf[r][s] = qp[2 * s];
    }
  }
  // compiler-visible: later waits then never hold for the copies in flight
  wait_vmcnt0_visible();

  // ---- copies (the layouts of fwd_wide.hpp): K instruction n (n = wave + 4 r,
  // r < SG / 4) fills 1 KiB of a dense half-tile, V^T instruction n (r < D / 64)
  // fills V^T rows 16 n .. 16 n + 15
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
    for (int r = 0; r < NKC; ++r) k_copy(tile, r, ln);
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
      kx[c] = (uint32_t)(KB + hf * HALF + r * (SG * 16) + (dense_pos(SG, r, 2 * c + hh) << 4));
  };
  // V^T fragment (A of O^T_half) for d-block db and 16-key step t2: row
  // W hf + 32 db + l % 32 of the tile, logical granule 2 t2 + l / 32 (vt_key order)
  auto v_bases = [&](int ln, uint32_t* vx) {
    const int r = ln & 31, hh = ln >> 5;
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      vx[t2] = (uint32_t)(VB + (W * hf + r) * 64 + (((2 * t2 + hh) ^ ((r >> 2) & 3)) << 4));
  };

  // ---- fp16 output accumulator: block (r, db) holds O^T[32 db .. +31][row]
  // of the lane's row as 16 packed fp16 (two u32x4: elements 0-7, 8-15 of the
  // MFMA C layout)
  u32x4 o16[RB][NDB][2];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int d = 0; d < NDB; ++d) o16[r][d][0] = o16[r][d][1] = u32x4{0, 0, 0, 0};
  float m_ref[RB], l_run[RB];  // reference max (log2 domain) and the full row sum
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    m_ref[r] = -INFINITY;
    l_run[r] = 0.f;
  }

  if (n_tiles > 0) issue_k_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    const int j0 = j * kWideBc;
    int lj = lane;
    asm volatile("" : "+v"(lj));
    const int hij = lj >> 5;

    // ===== K phase: partial S^T over this half for each row block
    wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    f32x16 s_acc[RB], s_odd;  // RB = 1: two chains (even / odd k-steps)
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
          if ((r * (NS / 2)) / NVC == st) vt_copy(j, r, vlo);
        const u32x4 a0 = kf[st % kKAhead];
        if (st + kKAhead < NS) kf[st % kKAhead] = kread(st + kKAhead);
        if constexpr (RB == 2) {
          if (st == 0) {
            mfma32_asm<BF16, true, false, true>(s_acc[0], a0, qf[0][st]);
            mfma32_asm<BF16, true, false, true>(s_acc[1], a0, qf[1][st]);
          } else if (st == NS - 1) {
            mfma32_asm<BF16, true, false>(s_acc[0], a0, qf[0][st]);
            mfma32_asm<BF16, true, false, false, false, true>(s_acc[1], a0, qf[1][st]);
          } else {
            mfma32_asm<BF16, true, false>(s_acc[0], a0, qf[0][st]);
            mfma32_asm<BF16, true, false>(s_acc[1], a0, qf[1][st]);
          }
        } else {
          f32x16& acc = (st & 1) ? s_odd : s_acc[0];
          if (st < 2) mfma32_asm<BF16, true, false, true>(acc, a0, qf[0][st]);
          else if (st == NS - 1) mfma32_asm<BF16, true, false, false, false, true>(acc, a0, qf[0][st]);
          else mfma32_asm<BF16, true, false>(acc, a0, qf[0][st]);
        }
      }
    }
    // every chain ends at least 19 wait states before this VALU (the last MFMA pads)
#pragma unroll
    for (int r = 0; r < RB; ++r) pin_after_pad(s_acc[r]);
    if constexpr (RB == 1) {
      pin_after_pad(s_odd);
#pragma unroll
      for (int i = 0; i < 16; ++i) s_acc[0][i] += s_odd[i];
    }

    // ===== swap partial scores with the other half's wave; add
    {
      FFPA_LDS f32x4* mine = (FFPA_LDS f32x4*)(smem + XB + wave * RB * kWideXchg) + lj;
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          mine[256 * r + 64 * jj] =
              f32x4{s_acc[r][4 * jj], s_acc[r][4 * jj + 1], s_acc[r][4 * jj + 2], s_acc[r][4 * jj + 3]};
      wait_lgkm0();
      barrier();
      const FFPA_LDS f32x4* other = (const FFPA_LDS f32x4*)(smem + XB + (wave ^ 1) * RB * kWideXchg) + lj;
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 x = other[256 * r + 64 * jj];
#pragma unroll
          for (int e = 0; e < 4; ++e) s_acc[r][4 * jj + e] += x[e];
        }
    }

    // ===== online softmax per row block (log2 domain), renormalised every
    // tile; register i of the scores holds key j0 + 8 (i / 4) + 4 hi + i % 4
    const int kb0 = j0 + 4 * hij;
    V8 pf[RB][2];
    float oscale[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int qw = qg + 32 * r;
      const int my_q = qw + (lj & 31);
      const bool need_mask = has_mask || (j0 + kWideBc > a.Nkv) || (a.causal && j0 + kWideBc - 1 > qw);
      float tv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tv[i] = s_acc[r][i] * a.scale_log2;
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
      if (__builtin_amdgcn_ballot_w64(mx > m_ref[r] + kRescaleTau) != 0) {  // wave-uniform
        const float m_new = fmaxf(m_ref[r], mx);
        alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_ref[r] - m_new);
        m_ref[r] = m_new;
      }
      const float m_use = (m_ref[r] == -INFINITY) ? 0.f : m_ref[r];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        tv[i] = exp2_fast(tv[i] - m_use);
        psum += tv[i];
      }
      const float l_old = l_run[r];
      const float l_new = alpha * l_old + psum + swap_halves(psum);
      l_run[r] = l_new;
      const float pscale = l_new > 0.f ? 1.f / l_new : 0.f;
      oscale[r] = alpha * l_old * pscale;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const float* x = &tv[8 * t2];
        pf[r][t2] = pack8<BF16>(x[0] * pscale, x[1] * pscale, x[2] * pscale, x[3] * pscale, x[4] * pscale,
                                x[5] * pscale, x[6] * pscale, x[7] * pscale);
      }
    }
    // P is the B operand of inline-asm MFMAs: every VALU write of it happens
    // here, before the barrier (the first MFMA of the phase pads as well)
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) asm volatile("" : "+v"(pf[r][t2]));

    // ===== V phase: per-tile products V_half^T P^T, folded into the fp16 O
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
      // unit u -> (d-block, row block); step s -> (group, unit of the group, t2)
      auto unit_db = [](int u) { return RB == 2 ? u >> 1 : u; };
      auto unit_r = [](int u) { return RB == 2 ? (u & 1) : 0; };
      auto step_of = [](int s, int& g, int& uu, int& t2) {
        g = s >> 2;
        const int k = s & 3;
        const bool pair = 2 * g + 1 < NU;
        uu = pair ? (k & 1) : 0;
        t2 = pair ? (k >> 1) : k;
      };
      // V^T fragment reads: RB = 2 shares one read between the two units of a
      // group (same d-block); RB = 1 reads one per step
      auto ev_of = [&](int s) {
        int g, uu, t2;
        step_of(s, g, uu, t2);
        return RB == 2 ? 2 * g + t2 : s;
      };
      constexpr int NEV = RB == 2 ? 2 * NG : NSV;
      auto vread_ev = [&](int e) {
        const int db = RB == 2 ? (e >> 1) : unit_db(2 * (e >> 2) + ((2 * (e >> 2) + 1 < NU) ? (e & 1) : 0));
        const int t2 = RB == 2 ? (e & 1) : ((2 * (e >> 2) + 1 < NU) ? ((e & 3) >> 1) : (e & 3));
        return lds_read16(smem + vx[t2] + 2048 * db);
      };
      u32x4 vf[kVAhead];
#pragma unroll
      for (int e = 0; e < kVAhead && e < NEV; ++e) vf[e] = vread_ev(e);

      f32x16 pv[2][2];  // [set = group % 2][unit of the group]
      auto fold_unit = [&](const f32x16& acc, int u) {
        const int db = unit_db(u), r = unit_r(u);
        const f16x2 sc = {(_Float16)oscale[r], (_Float16)oscale[r]};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4 w = o16[r][db][hh];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f16x2 cur = f16x2_from_bits(w[e]);
            const f16x2 add = {(_Float16)acc[8 * hh + 2 * e], (_Float16)acc[8 * hh + 2 * e + 1]};
            cur = cur * sc + add;
            w[e] = __builtin_bit_cast(uint32_t, cur);
          }
          o16[r][db][hh] = w;
        }
      };
      auto fold_group = [&](int g) {
        fold_unit(pv[g & 1][0], 2 * g);
        if (2 * g + 1 < NU) fold_unit(pv[g & 1][1], 2 * g + 1);
        // the folded values exist here, before the next MFMAs (which reuse
        // this set's registers two groups later)
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          if (2 * g + uu >= NU) continue;
          const int db = unit_db(2 * g + uu), r = unit_r(2 * g + uu);
          asm volatile("" : "+v"(o16[r][db][0]), "+v"(o16[r][db][1]));
        }
      };
      int lnc = lane;
      asm volatile("" : "+v"(lnc));
#pragma unroll
      for (int s = 0; s < NSV; ++s) {
        // K(j+1); on the last tile rows past the key range (range-checked
        // zeros) or, causal, rows nobody reads: harmless, and branch-free
#pragma unroll
        for (int r = 0; r < NKC; ++r)
          if ((r * (NSV / 2)) / NKC == s) k_copy(j + 1, r, lnc);
        int g, uu, t2;
        step_of(s, g, uu, t2);
        const int u = 2 * g + uu;
        const int e = ev_of(s);
        const u32x4 vbits = vf[e % kVAhead];
        // the last use of event e: read e + kVAhead into its slot
        const bool last_use = RB == 2 ? (uu == 1 || 2 * g + 1 >= NU) : true;
        if (last_use && e + kVAhead < NEV) vf[e % kVAhead] = vread_ev(e + kVAhead);
        const u32x4 pb = __builtin_bit_cast(u32x4, pf[unit_r(u)][t2]);
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

  // ===== epilogue: each row block's rows of the half go through LDS (32 rows
  // per wave, pitch of whole 16-granule groups), then out as contiguous pieces
  // of W elements per row
  constexpr int PITCH = wide16_pitch<D>();  // bytes per staged row
  static_assert(4 * 32 * PITCH <= wide16_lds<D>(), "epilogue staging fits the LDS");
  wait_lgkm0();
  barrier();  // every wave is done with the tile buffers
  FFPA_LDS char* ostage = smem + wave * 32 * PITCH;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    const int qw = qg + 32 * r;
    {
      const int rr = lane & 31, hie = lane >> 5;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x4 w = o16[r][db][g4 >> 1];
          const f16x2 p0 = f16x2_from_bits(w[2 * (g4 & 1)]);
          const f16x2 p1 = f16x2_from_bits(w[2 * (g4 & 1) + 1]);
          const u32x2 st = {E::pack2((float)p0[0], (float)p0[1]), E::pack2((float)p1[0], (float)p1[1])};
          const int gg = 4 * db + g4;  // elements 32 db + 8 g4 + 4 hi .. +3
          *(FFPA_LDS u32x2*)(ostage + rr * PITCH + ((gg ^ (rr & 15)) << 4) + 8 * hie) = st;
        }
    }
    {
      typename E::scalar* O = (typename E::scalar*)a.o + ((size_t)(b * a.Hq + h) * a.Nq + qw) * D + W * hf;
      const int rows = min(32, a.Nq - qw);
      constexpr int NIT = (32 * SG + 63) / 64;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int c = it * 64 + lane;
        const int rr = c / SG, gg = c % SG;
        if (rr < rows) {
          const u32x4 x = *(const FFPA_LDS u32x4*)(ostage + rr * PITCH + ((gg ^ (rr & 15)) << 4));
          *(u32x4*)(O + (size_t)rr * D + 8 * gg) = x;
        }
      }
    }
    if (hf == 0 && a.lse != nullptr && (lane >> 5) == 0 && qw + lane < a.Nq) {
      float* L = a.lse + (size_t)(b * a.Hq + h) * a.Nq + qw + lane;
      *L = l_run[r] > 0.f ? (m_ref[r] + __builtin_amdgcn_logf(l_run[r])) * kLn2 : -INFINITY;
    }
  }
}

// Host launcher: the transposed copy of V (blocks of 32 keys) into a.vt, then
// the kernel over ceil(Nq / wide16_rows<D>()) row blocks per head. The LDS
// limit is set before anything is enqueued.
template <int D, bool BF16>
hipError_t launch_fwd_wide16(const FwdArgs& a, hipStream_t stream) {
  auto kern = fwd_wide16_kernel<D, BF16>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, wide16_lds<D>());
  if (attr != hipSuccess) return attr;
  const hipError_t e = launch_fwd_vt(a.v, const_cast<void*>(a.vt), a.B * a.Hkv, a.Nkv, D, kWideBc, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.total_wg), dim3(256), wide16_lds<D>(), stream, a);
  return hipGetLastError();
}

}  // namespace ffpa
