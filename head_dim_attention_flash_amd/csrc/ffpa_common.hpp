// Shared device helpers for the gfx950 (CDNA4) attention kernels:
// vector types, MFMA wrappers, the LDS swizzle, direct global->LDS copies,
// explicit wait counters and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffpa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FFPA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element traits: fp16 or bf16 storage, fp32 MFMA accumulation.
// MFMA v_mfma_f32_32x32x16_{f16,bf16} lane layout (checked on gfx950):
//   A[m][k]: lane l holds m = l % 32, k = 8 * (l / 32) + e, e = 0..7
//   B[k][n]: lane l holds k = 8 * (l / 32) + e, n = l % 32
//   C[m][n]: lane l, reg i holds m = 8 * (i / 4) + 4 * (l / 32) + i % 4, n = l % 32
// v_mfma_f32_16x16x32_{f16,bf16}:
//   A[m][k]: m = l % 16, k = 8 * (l / 16) + e;  B[k][n]: k = 8 * (l / 16) + e, n = l % 16
//   C[m][n]: lane l, reg i holds m = 4 * (l / 16) + i, n = l % 16
// ---------------------------------------------------------------------------
template <bool BF16>
struct Elem;

template <>
struct Elem<false> {
  using scalar = _Float16;
  using vec8 = f16x8;
  __device__ static inline f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline float to_f32(uint16_t bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
  // Round-to-nearest-even pack of two floats.
  __device__ static inline uint32_t pack2(float a, float b) {
    f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
  }
};

template <>
struct Elem<true> {
  using scalar = __bf16;
  using vec8 = bf16x8;
  __device__ static inline f32x16 mfma32(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline float to_f32(uint16_t bits) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  }
  // Round-to-nearest-even pack of two floats: one v_cvt_pk_bf16_f32 (two
  // scalar conversions compile to two of them plus a shift and an or).
  __device__ static inline uint32_t pack2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
  }
};

// Two fp16 values from their packed bits. Takes the word BY VALUE: this clang
// mis-lowers __builtin_bit_cast applied directly to an ext_vector element
// (every element of the vector then reads as element 0).
__device__ inline f16x2 f16x2_from_bits(uint32_t bits) { return __builtin_bit_cast(f16x2, bits); }

// ---------------------------------------------------------------------------
// MFMA 32x32x16 issued as inline asm so that operand register files can be
// chosen (the compiler will not feed an MFMA source from AGPRs by itself):
// A in VGPRs, B in AGPRs (B_A) or VGPRs (B_V), C/D in AGPRs (C_A) or VGPRs
// (C_V). The compiler does not know these are MFMAs, so hazards it would
// otherwise pad are handled here:
//  - an MFMA result read by a VALU or accvgpr instruction needs up to 19 wait
//    states: the last MFMA of a chain is issued with mfma_last=true (pads 21);
//  - a VALU write of an MFMA source needs a few wait states: a chain whose B
//    operand was just written by VALU code starts with mfma_first=true (pads 4).
// Back-to-back MFMAs whose C is exactly the previous D are interlocked by the
// hardware. `zero` replaces C by the inline constant 0.
// ---------------------------------------------------------------------------
#define FFPA_MFMA_ASM(OPC, CA, BA, ZERO, PRE, POST)                                            \
  if constexpr (ZERO)                                                                           \
    asm volatile(PRE OPC " %0, %1, %2, 0" POST : "=&" CA(acc) : "v"(a), BA(b));                 \
  else                                                                                          \
    asm volatile(PRE OPC " %0, %1, %2, %0" POST : "+" CA(acc) : "v"(a), BA(b));
template <bool BF16, bool B_AGPR, bool C_AGPR, bool ZERO = false, bool FIRST = false, bool LAST = false>
__device__ inline void mfma32_asm(f32x16& acc, u32x4 a, u32x4 b) {
#define FFPA_PRE (FIRST ? "s_nop 4\n" : "")
  // PRE/POST must be string literals: select with constexpr branches
  if constexpr (!BF16) {
    if constexpr (FIRST && LAST) {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "a", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "a", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "v", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "v", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    } else if constexpr (FIRST) {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "a", ZERO, "s_nop 4\n", "") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "a", ZERO, "s_nop 4\n", "") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "v", ZERO, "s_nop 4\n", "") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "v", ZERO, "s_nop 4\n", "") }
    } else if constexpr (LAST) {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "a", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "a", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "v", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "v", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    } else {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "a", ZERO, "", "") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "a", ZERO, "", "") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "a", "v", ZERO, "", "") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_f16", "v", "v", ZERO, "", "") }
    }
  } else {
    if constexpr (FIRST && LAST) {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "a", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "a", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "v", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "v", ZERO, "s_nop 4\n", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    } else if constexpr (FIRST) {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "a", ZERO, "s_nop 4\n", "") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "a", ZERO, "s_nop 4\n", "") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "v", ZERO, "s_nop 4\n", "") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "v", ZERO, "s_nop 4\n", "") }
    } else if constexpr (LAST) {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "a", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "a", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "v", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "v", ZERO, "", "\n s_nop 7\n s_nop 7\n s_nop 4") }
    } else {
      if constexpr (B_AGPR && C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "a", ZERO, "", "") }
      else if constexpr (B_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "a", ZERO, "", "") }
      else if constexpr (C_AGPR) { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "a", "v", ZERO, "", "") }
      else { FFPA_MFMA_ASM("v_mfma_f32_32x32x16_bf16", "v", "v", ZERO, "", "") }
    }
  }
#undef FFPA_PRE
}
#undef FFPA_MFMA_ASM

// Orders every later read of `acc` after this point. Used after an MFMA chain
// that ends padded (LAST) on a sibling accumulator: the compiler would
// otherwise be free to move a VALU read of `acc`, whose own last MFMA is
// earlier, above that padding.
__device__ inline void pin_after_pad(f32x16& acc) { asm volatile("" : "+v"(acc)); }

// A compile-time boolean as a type, to instantiate a generic lambda twice.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

template <class V>
__device__ inline V as_vec8(u32x4 x) {
  return __builtin_bit_cast(V, x);
}

// Eight packed 16-bit values from eight floats (round to nearest even).
template <bool BF16>
__device__ inline typename Elem<BF16>::vec8 pack8(float a0, float a1, float a2, float a3, float a4,
                                                   float a5, float a6, float a7) {
  u32x4 w = {Elem<BF16>::pack2(a0, a1), Elem<BF16>::pack2(a2, a3), Elem<BF16>::pack2(a4, a5),
             Elem<BF16>::pack2(a6, a7)};
  return __builtin_bit_cast(typename Elem<BF16>::vec8, w);
}

// ---------------------------------------------------------------------------
// LDS tiles. A staged tile is R rows of D 16-bit values (rows of 2D bytes,
// 16-byte granules). The LDS serves 64 banks of 4 bytes: a 16-byte read is
// conflict-free when the 16 lanes served together hit 16 distinct 16-byte
// slots modulo 256 bytes, an 8-byte read when 32 lanes hit distinct 8-byte
// slots. Within every complete group of 16 granules of a row, granule g of
// row r is stored at g ^ swz4(r); a trailing group of 8 granules (D % 128 ==
// 64) uses the low three bits of swz4(r). This makes both access patterns of
// the attention kernels conflict-free for D % 128 == 0 (and leaves at most
// two-way conflicts in the trailing group otherwise):
//  - 16 consecutive rows reading the same granule (K fragments, b128), and
//  - 4 consecutive rows x 4 consecutive granules (one half-wave of transposed
//    V^T reads, ds_read_b64_tr_b16).
// ---------------------------------------------------------------------------
__device__ __host__ inline int swz4(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

// Stored position of logical granule g of row r in a staged tile of dense
// rows, P granules (16 bytes) each, P a multiple of 4: XOR swizzle inside
// aligned groups of 16, 8 or 4 granules chosen by P % 16, so that sixteen
// lanes reading the same logical granule of sixteen consecutive rows hit
// distinct banks whatever the pitch. An involution: it also maps a stored
// position back to its logical granule.
__device__ __host__ inline int dense_pos(int P, int r, int g) {
  const int m = P % 16;
  const int G = m == 0 ? 16 : (m == 8 ? 8 : 4);
  const int x = m == 0 ? swz4(r) : (m == 8 ? (r >> 1) & 7 : (r >> 2) & 3);
  return (g & ~(G - 1)) | ((g & (G - 1)) ^ x);
}

// Stored granule of logical granule g of row `row` (and, the map being an
// involution within each group, the logical granule of stored granule g).
template <int GPR>
__device__ __host__ inline int swz_granule(int row, int g) {
  return ((g & ~15) + 16 <= GPR) ? (g ^ swz4(row)) : (g ^ (swz4(row) & 7));
}

// ---------------------------------------------------------------------------
// Wait counters and the workgroup barrier, as inline asm with a "memory"
// clobber: the compiler must not move any load or store (LDS reads of a
// chunk, copies into a slot) across them. The clang builtins for these
// instructions are not memory barriers.
// ---------------------------------------------------------------------------
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// vmcnt(0) that the compiler's wait-count pass sees (the builtin, not asm):
// after it the pass knows every earlier vector-memory load has landed and
// inserts no further waits for them. Used after a kernel's prologue loads of
// registers that the main loop only reads; without it the pass keeps waiting
// for them inside the loop, where its counts cannot see the asm copies, and
// those waits then also hold for the copies in flight.
__device__ inline void wait_vmcnt0_visible() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ inline void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Buffer resource over `bytes` bytes at `base` (raw, stride 0). Loads at or
// past `bytes` return zero instead of touching memory. 0x00020000 selects the
// 32-bit data format gfx9 requires of untyped buffer loads.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16-byte direct copy buffer -> LDS: lane t of the wave reads
// rsrc[voff .. +16) and writes LDS bytes [16 t, 16 t + 16) after `lds_base`
// (wave-uniform, passed in M0). The range check applies to voff: reads with
// voff at or past the range write zeros.
//
// Issued as inline asm on purpose. The compiler's wait-count pass treats a
// copy into LDS it knows about as a pending LDS write, and when it cannot
// prove that a later LDS read touches another buffer it waits for every
// outstanding copy (s_waitcnt vmcnt(0)) before that read: a full memory
// latency per tile. The kernels order copies and reads themselves
// (wait_vmcnt before the barrier that publishes a tile), so the copy is kept
// out of the compiler's tracking.
//
// The compiler does not pad hazards for inline asm either. s_nop 0 covers
// the M0 write -> LDS copy hazard. The scalar offset is the constant 0, so the
// only SGPRs read are the resource and M0; a VALU write of one of them (a
// v_readlane restoring a spilled SGPR) would need 5 wait states before the
// copy. The compiler has no reason to place one there, and the static hazard
// check of the built kernels (check_hazards.py, run by the CPU test suite)
// rejects a build where it does: copies issue every few MFMAs, so a longer
// fixed pad would cost throughput for nothing.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, FFPA_LDS void* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)lds_base;
  asm volatile("s_nop 0\n buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(m0)
               : "memory");
}

__device__ inline u32x4 lds_read16(const FFPA_LDS char* p) { return *(const FFPA_LDS u32x4*)p; }

// Four consecutive entries k4 .. k4 + 3 (k4 a multiple of 4) of one row of an
// additive mask in the 16-bit input type, as floats; entries at or past Nkv
// read as 0 (the callers mask those keys anyway) and are never loaded. With
// Nkv % 4 == 0 a group is wholly inside or outside the row and is one 8-byte
// load; otherwise each entry is loaded on its own, clamped.
template <bool BF16>
__device__ inline f32x4 mask_row4(const uint16_t* row, int k4, int nkv, bool by8) {
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
  if (by8) {
    if (k4 < nkv) {
      const u32x2 w = *(const u32x2*)(row + k4);
      r = f32x4{Elem<BF16>::to_f32((uint16_t)(w[0] & 0xffff)), Elem<BF16>::to_f32((uint16_t)(w[0] >> 16)),
                Elem<BF16>::to_f32((uint16_t)(w[1] & 0xffff)), Elem<BF16>::to_f32((uint16_t)(w[1] >> 16))};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = k4 + e;
      const float x = Elem<BF16>::to_f32(row[min(k, nkv - 1)]);
      r[e] = k < nkv ? x : 0.f;
    }
  }
  return r;
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, lane j receives element (j % 4) of the 4-element chunks addressed by
// lanes j/4, j/4 + 4, j/4 + 8 and j/4 + 12 (in that order). Checked on gfx950.
__device__ inline i16x4 lds_read_tr(const FFPA_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FFPA_LDS i16x4*)p);
}

__device__ inline u32x4 join8(i16x4 lo, i16x4 hi) {
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(u32x4, v);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// acc *= s for a 16-float MFMA accumulator that lives in AGPRs: each value
// goes AGPR -> VGPR -> multiply -> AGPR through one VGPR temporary, so the
// accumulator never has to be copied out as a whole. The s_nop padding covers
// the MFMA-write -> accvgpr-read and accvgpr-write -> MFMA-read hazards, which
// the compiler cannot see inside inline asm.
#define FFPA_RESCALE1(i) \
  "v_accvgpr_read_b32 %[t], %[a" #i "]\n v_mul_f32 %[t], %[s], %[t]\n v_accvgpr_write_b32 %[a" #i "], %[t]\n"
__device__ inline void scale_agpr16(f32x16& acc, float s) {
  float x0 = acc[0], x1 = acc[1], x2 = acc[2], x3 = acc[3], x4 = acc[4], x5 = acc[5], x6 = acc[6],
        x7 = acc[7], x8 = acc[8], x9 = acc[9], x10 = acc[10], x11 = acc[11], x12 = acc[12],
        x13 = acc[13], x14 = acc[14], x15 = acc[15];
  float t;
  asm volatile("s_nop 7\n s_nop 7\n s_nop 4\n" FFPA_RESCALE1(0) FFPA_RESCALE1(1) FFPA_RESCALE1(2)
                   FFPA_RESCALE1(3) FFPA_RESCALE1(4) FFPA_RESCALE1(5) FFPA_RESCALE1(6)
                       FFPA_RESCALE1(7) FFPA_RESCALE1(8) FFPA_RESCALE1(9) FFPA_RESCALE1(10)
                           FFPA_RESCALE1(11) FFPA_RESCALE1(12) FFPA_RESCALE1(13)
                               FFPA_RESCALE1(14) FFPA_RESCALE1(15) "s_nop 7\n s_nop 7\n"
               : [a0] "+a"(x0), [a1] "+a"(x1), [a2] "+a"(x2), [a3] "+a"(x3), [a4] "+a"(x4),
                 [a5] "+a"(x5), [a6] "+a"(x6), [a7] "+a"(x7), [a8] "+a"(x8), [a9] "+a"(x9),
                 [a10] "+a"(x10), [a11] "+a"(x11), [a12] "+a"(x12), [a13] "+a"(x13),
                 [a14] "+a"(x14), [a15] "+a"(x15), [t] "=&v"(t)
               : [s] "v"(s));
  acc = f32x16{x0, x1, x2, x3, x4, x5, x6, x7, x8, x9, x10, x11, x12, x13, x14, x15};
}
#undef FFPA_RESCALE1

// ---------------------------------------------------------------------------
// Dropout's random numbers: the counter-based generator Philox-4x32-10
// (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
// 3", SC 2011). Each of its 10 rounds multiplies two counter words by fixed
// odd constants, recombines the halves of the 64-bit products with the other
// two words and the key, and bumps the key by two further constants. One call
// serves a block of 4 query rows x 4 keys of a head: counter (key / 4,
// query / 4, b * Hq + h, 0) under the 64-bit seed; element (query, key) is the
// byte key % 4 of output word query % 4, kept when it is >= t.
// ---------------------------------------------------------------------------
struct DropParams {
  uint32_t t;        // threshold: 0 = no dropout; else round(256 p), 1 .. 255
  uint32_t seed_lo;  // key words
  uint32_t seed_hi;
  float scale;       // 256 / (256 - t): the scale of a kept element
};

__device__ inline u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                      uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// The four dropout bytes of query row q for keys k4 .. k4 + 3 (k4 a multiple
// of 4) of head bh, one per byte (key k4 + e in byte e).
__device__ inline uint32_t drop_row_word(const DropParams& d, int bh, int q, int k4) {
  const u32x4 w = philox4x32_10((uint32_t)k4 >> 2, (uint32_t)q >> 2, (uint32_t)bh, 0u, d.seed_lo, d.seed_hi);
  const int r = q & 3;
  return r == 0 ? w[0] : r == 1 ? w[1] : r == 2 ? w[2] : w[3];
}

// Whether byte e of a dropout word keeps its element.
__device__ inline bool drop_keeps(uint32_t word, int e, uint32_t t) { return ((word >> (8 * e)) & 0xffu) >= t; }

// Keep bits of one generator call: bit 4 r + e = byte e of word r kept
// (query 4 c1 + r, key 4 c0 + e).
__device__ inline uint32_t drop_block_bits(const u32x4 w, uint32_t t) {
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) m |= (uint32_t)drop_keeps(w[r], e, t) << (4 * r + e);
  return m;
}

// Value of x in lane j of this lane's quad (lanes 4 a .. 4 a + 3).
template <int J>
__device__ inline uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, J * 0x55, 0xf, 0xf, false);
}

// The four lanes of a quad hold four consecutive 4-aligned positions of one
// orientation and need the same four generator calls; lane j of the quad
// makes call j and the others read its 16 bits. Every lane of the wave must
// be active.
//
// Row per lane (lane & 3 == q & 3): keep bits of query q against keys
// k0 + 8 j + e (k0 a multiple of 4), bit 4 j + e.
__device__ inline uint32_t drop_bits_row(const DropParams& d, int bh, int q, int k0) {
  // opaque inputs: nothing of the call (the per-round keys included) is
  // hoisted out of the caller's loop, where it would hold registers
  uint32_t s0 = d.seed_lo, s1 = d.seed_hi;
  asm volatile("" : "+v"(q), "+s"(s0), "+s"(s1));
  const int r = q & 3;  // this lane's index in its quad
  const uint32_t m = drop_block_bits(
      philox4x32_10((uint32_t)(k0 + 8 * r) >> 2, (uint32_t)q >> 2, (uint32_t)bh, 0u, s0, s1), d.t);
  const int sh = 4 * r;
  uint32_t keep = ((quad_bcast<0>(m) >> sh) & 0xfu) | (((quad_bcast<1>(m) >> sh) & 0xfu) << 4) |
                  (((quad_bcast<2>(m) >> sh) & 0xfu) << 8) | (((quad_bcast<3>(m) >> sh) & 0xfu) << 12);
  asm volatile("" : "+v"(keep));  // finished here: one register stays live, not four
  return keep;
}

// Key per lane (lane & 3 == k & 3): keep bits of key k against queries
// q0 + 8 j + e (q0 a multiple of 4), bit 4 j + e.
__device__ inline uint32_t drop_bits_col(const DropParams& d, int bh, int k, int q0) {
  uint32_t s0 = d.seed_lo, s1 = d.seed_hi;
  asm volatile("" : "+v"(k), "+s"(s0), "+s"(s1));  // opaque inputs, as in drop_bits_row
  const int r = k & 3;  // this lane's index in its quad
  const uint32_t m = drop_block_bits(
      philox4x32_10((uint32_t)k >> 2, (uint32_t)(q0 + 8 * r) >> 2, (uint32_t)bh, 0u, s0, s1), d.t);
  auto gather = [r](uint32_t mj) {  // bits r, 4 + r, 8 + r, 12 + r -> 0..3
    uint32_t x = (mj >> r) & 0x1111u;
    x |= x >> 3;
    return (x | (x >> 6)) & 0xfu;
  };
  uint32_t keep = gather(quad_bcast<0>(m)) | (gather(quad_bcast<1>(m)) << 4) | (gather(quad_bcast<2>(m)) << 8) |
                  (gather(quad_bcast<3>(m)) << 12);
  asm volatile("" : "+v"(keep));  // finished here: one register stays live, not four
  return keep;
}

// x where bit b (0..15) of `bits` is set, else +0. The bit-field extract and
// the AND sit in one asm block, so the all-ones/zero mask lives only inside
// it (the compiler's scheduler would otherwise make the 16 masks of a tile at
// once, 16 registers where the kernels have none to spare). b is a constant
// in unrolled callers, where the switch folds away.
__device__ inline float keep_if_bit(float x, uint32_t bits, int b) {
  float r = 0.f;
  uint32_t m;
#define FFPA_KEEP_BIT(B)                                                                                    \
  case B:                                                                                                   \
    asm("v_bfe_i32 %1, %2, " #B ", 1\n\tv_and_b32 %0, %3, %1" : "=v"(r), "=&v"(m) : "v"(bits), "v"(x)); \
    break;
  switch (b) {
    FFPA_KEEP_BIT(0) FFPA_KEEP_BIT(1) FFPA_KEEP_BIT(2) FFPA_KEEP_BIT(3)
    FFPA_KEEP_BIT(4) FFPA_KEEP_BIT(5) FFPA_KEEP_BIT(6) FFPA_KEEP_BIT(7)
    FFPA_KEEP_BIT(8) FFPA_KEEP_BIT(9) FFPA_KEEP_BIT(10) FFPA_KEEP_BIT(11)
    FFPA_KEEP_BIT(12) FFPA_KEEP_BIT(13) FFPA_KEEP_BIT(14) FFPA_KEEP_BIT(15)
    default: break;
  }
#undef FFPA_KEEP_BIT
  return r;
}

// Value of lane (l ^ 32) of x.
__device__ inline float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// ---------------------------------------------------------------------------
// Workgroup order. The dispatcher hands workgroup i to XCD i % 8; each XCD has
// its own L2. Logical tile t is given to workgroup ids so that every XCD works
// on a contiguous range of logical tiles (tiles of the same head share K/V in
// that XCD's L2).
// ---------------------------------------------------------------------------
__device__ inline int xcd_logical(int bid, int total) {
  constexpr int kXcd = 8;
  int x = bid % kXcd, j = bid / kXcd;
  int per = total / kXcd, rem = total % kXcd;
  return x * per + (x < rem ? x : rem) + j;
}

// Causal passes: logical tile t (xcd_logical order) -> position p of its
// block in longest-first order within head t / nblk. A head whose blocks fill
// several XCD ranges exactly (the range of total / 8 tiles divides nblk)
// would give the first XCD its longest blocks and the last its shortest; XCD
// r of the s that share the head takes positions r, r + s, r + 2 s, ...
// instead, so every XCD gets an even share of the triangle, longest first.
__device__ inline int causal_position(int t, int nblk, int total) {
  int p = t % nblk;
  if (total % 8 == 0) {
    const int per = total / 8;
    if (per < nblk && nblk % per == 0) p = (p % per) * (nblk / per) + p / per;
  }
  return p;
}

}  // namespace ffpa
