// C ABI of libffpa_attn: argument validation, kernel selection and launch.
// The operation and its conventions are documented in include/ffpa_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <string>

#include "ffpa_attn.h"
#include "bwd.hpp"
#include "dec_bwd.hpp"
#include "decode.hpp"
#include "fwd_fp8.hpp"
#include "fwd_prefill.hpp"
#include "fwd_vt.hpp"
#include "fwd_wide.hpp"
#include "fwd_wide16.hpp"
#include "instances.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

constexpr size_t kLdsLimit = 160 * 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

using FwdLauncher = hipError_t (*)(const ffpa::FwdArgs&, size_t, hipStream_t);

template <int D, bool VT>
FwdLauncher pick_fwd(int bf16, int acc16, bool drop) {
  // dropout is built with the fp32 accumulator (the caller has checked)
  if (drop) return bf16 ? ffpa::launch_fwd_prefill<D, true, false, VT, true> : ffpa::launch_fwd_prefill<D, false, false, VT, true>;
  if (bf16) return acc16 ? ffpa::launch_fwd_prefill<D, true, true, VT> : ffpa::launch_fwd_prefill<D, true, false, VT>;
  return acc16 ? ffpa::launch_fwd_prefill<D, false, true, VT> : ffpa::launch_fwd_prefill<D, false, false, VT>;
}

FwdLauncher fwd_launcher(int D, int bf16, int acc16, bool vt, bool drop, size_t* ring_bytes) {
  switch (D) {
#define FFPA_CASE(DD)                                                  \
  case DD:                                                             \
    *ring_bytes = ffpa::fwd_ring_bytes<DD>();                          \
    return vt ? pick_fwd<DD, true>(bf16, acc16, drop) : pick_fwd<DD, false>(bf16, acc16, drop);
    FFPA_CASE(64)
    FFPA_CASE(128)
    FFPA_CASE(192)
    FFPA_CASE(256)
    FFPA_CASE(320)
    FFPA_CASE(384)
    FFPA_CASE(448)
    FFPA_CASE(512)
#undef FFPA_CASE
    // 576 and 640: the fp16 accumulator with V^T staged only (the one-part
    // tile shape of the wide forward)
#define FFPA_CASE(DD)                                                                                  \
  case DD:                                                                                             \
    *ring_bytes = ffpa::fwd_ring_bytes<DD>();                                                          \
    if (!acc16 || !vt || drop) return nullptr;                                                         \
    return bf16 ? ffpa::launch_fwd_prefill<DD, true, true, true> : ffpa::launch_fwd_prefill<DD, false, true, true>;
    FFPA_CASE(576)
    FFPA_CASE(640)
#undef FFPA_CASE
    default:
      return nullptr;
  }
}

using WideLauncher = hipError_t (*)(const ffpa::FwdArgs&, hipStream_t);

// The wide kernels (D > 512), by tile shape:
//   kWideF32:   fwd_wide_kernel, fp32 output accumulator, 64 rows per workgroup;
//   kWide16One: fp16 accumulator, a wave holds all of D, 128 rows per
//               workgroup (D <= 768 only): fwd_wide16_kernel at 704 and 768,
//               the prefill kernel (64-key tiles) at 576 and 640;
//   kWide16Two: fwd_wide16_kernel, fp16 accumulator, a wave pair splits D,
//               64 rows per workgroup.
enum WideShape { kWideF32 = 1, kWide16One = 2, kWide16Two = 3 };

WideLauncher wide_launcher(int D, int bf16, int shape, bool drop, int* rows) {
  switch (D) {
#define FFPA_CASE(DD)                                                                                  \
  case DD:                                                                                             \
    if (drop || shape == kWideF32) {                                                                   \
      *rows = 64;                                                                                      \
      if (drop) return bf16 ? ffpa::launch_fwd_wide<DD, true, true> : ffpa::launch_fwd_wide<DD, false, true>; \
      return bf16 ? ffpa::launch_fwd_wide<DD, true> : ffpa::launch_fwd_wide<DD, false>;               \
    }                                                                                                  \
    if (shape == kWide16Two) {                                                                         \
      *rows = ffpa::wide16_rows<DD, 2>();                                                              \
      return bf16 ? ffpa::launch_fwd_wide16<DD, true, 2> : ffpa::launch_fwd_wide16<DD, false, 2>;     \
    }                                                                                                  \
    if (DD > 768) return nullptr;                                                                      \
    *rows = ffpa::wide16_rows<DD, 1>();                                                                \
    return bf16 ? ffpa::launch_fwd_wide16<DD, true, 1> : ffpa::launch_fwd_wide16<DD, false, 1>;
    FFPA_CASE(704) FFPA_CASE(768)
#undef FFPA_CASE
#define FFPA_CASE(DD)                                                                                  \
  case DD:                                                                                             \
    if (drop || shape == kWideF32) {                                                                   \
      *rows = 64;                                                                                      \
      if (drop) return bf16 ? ffpa::launch_fwd_wide<DD, true, true> : ffpa::launch_fwd_wide<DD, false, true>; \
      return bf16 ? ffpa::launch_fwd_wide<DD, true> : ffpa::launch_fwd_wide<DD, false>;               \
    }                                                                                                  \
    if (shape != kWide16Two) return nullptr; /* kWide16One: the prefill kernel */                      \
    *rows = ffpa::wide16_rows<DD, 2>();                                                                \
    return bf16 ? ffpa::launch_fwd_wide16<DD, true, 2> : ffpa::launch_fwd_wide16<DD, false, 2>;
    FFPA_CASE(576) FFPA_CASE(640)
#undef FFPA_CASE
#define FFPA_CASE(DD)                                                                                  \
  case DD:                                                                                             \
    if (drop || shape == kWideF32) {                                                                   \
      *rows = 64;                                                                                      \
      if (drop) return bf16 ? ffpa::launch_fwd_wide<DD, true, true> : ffpa::launch_fwd_wide<DD, false, true>; \
      return bf16 ? ffpa::launch_fwd_wide<DD, true> : ffpa::launch_fwd_wide<DD, false>;               \
    }                                                                                                  \
    if (shape != kWide16Two) return nullptr;                                                           \
    *rows = ffpa::wide16_rows<DD, 2>();                                                                \
    return bf16 ? ffpa::launch_fwd_wide16<DD, true, 2> : ffpa::launch_fwd_wide16<DD, false, 2>;
    FFPA_CASE(832) FFPA_CASE(896) FFPA_CASE(960) FFPA_CASE(1024)
#undef FFPA_CASE
    default:
      return nullptr;
  }
}

using Fp8Launcher = hipError_t (*)(const ffpa::Fp8Args&, hipStream_t);

Fp8Launcher fp8_launcher(int D, int bf16) {
  switch (D) {
#define FFPA_CASE(DD) \
  case DD:            \
    return bf16 ? ffpa::launch_fwd_fp8<DD, true> : ffpa::launch_fwd_fp8<DD, false>;
    FFPA_CASE(128) FFPA_CASE(192) FFPA_CASE(256) FFPA_CASE(320) FFPA_CASE(384) FFPA_CASE(448) FFPA_CASE(512)
#undef FFPA_CASE
    default:
      return nullptr;
  }
}

using DecLauncher = hipError_t (*)(const ffpa::DecArgs&, hipStream_t);

DecLauncher dec_launcher(int D, int bf16) {
  switch (D) {
#define FFPA_CASE(DD) \
  case DD:            \
    return bf16 ? ffpa::launch_decode<DD, true> : ffpa::launch_decode<DD, false>;
    FFPA_CASE(32) FFPA_CASE(64) FFPA_CASE(96) FFPA_CASE(128) FFPA_CASE(160) FFPA_CASE(192)
    FFPA_CASE(224) FFPA_CASE(256) FFPA_CASE(288) FFPA_CASE(320) FFPA_CASE(352) FFPA_CASE(384)
    FFPA_CASE(416) FFPA_CASE(448) FFPA_CASE(480) FFPA_CASE(512) FFPA_CASE(544) FFPA_CASE(576)
    FFPA_CASE(608) FFPA_CASE(640) FFPA_CASE(672) FFPA_CASE(704) FFPA_CASE(736) FFPA_CASE(768)
    FFPA_CASE(800) FFPA_CASE(832) FFPA_CASE(864) FFPA_CASE(896) FFPA_CASE(928) FFPA_CASE(960)
    FFPA_CASE(992) FFPA_CASE(1024)
#undef FFPA_CASE
    default:
      return nullptr;
  }
}

// Keys a decode row sees: top-left causal leaves row 0 only key 0.
int dec_kv_end(int Nkv, int causal) { return causal ? 1 : Nkv; }

using BwdLauncher = hipError_t (*)(const ffpa::BwdArgs&, int, hipStream_t);

BwdLauncher bwd_launcher(int D, int bf16) {
  switch (D) {
#define FFPA_CASE(DD) \
  case DD:            \
    return bf16 ? ffpa::launch_bwd<DD, true> : ffpa::launch_bwd<DD, false>;
    FFPA_CASE(64)
    FFPA_CASE(128)
    FFPA_CASE(192)
    FFPA_CASE(256)
    FFPA_CASE(320)
    FFPA_CASE(384)
    FFPA_CASE(448)
    FFPA_CASE(512)
    FFPA_CASE(576)
    FFPA_CASE(640)
    FFPA_CASE(704)
    FFPA_CASE(768)
    FFPA_CASE(832)
    FFPA_CASE(896)
    FFPA_CASE(960)
    FFPA_CASE(1024)
#undef FFPA_CASE
    default:
      return nullptr;
  }
}

using DecBwdLauncher = hipError_t (*)(const ffpa::DecBwdArgs&, hipStream_t);

// The decode backward (Nq = 1) by head dimension and group size G = Hq / Hkv:
// built for D = 64 .. 1024 (step 64), G = 1, 2, 4 up to D = 512 and G = 1, 2
// above; nullptr otherwise.
template <int D>
DecBwdLauncher dec_bwd_pick(int bf16, int G) {
  if (G == 1) return bf16 ? ffpa::launch_dec_bwd<D, true, 1> : ffpa::launch_dec_bwd<D, false, 1>;
  if (G == 2) return bf16 ? ffpa::launch_dec_bwd<D, true, 2> : ffpa::launch_dec_bwd<D, false, 2>;
  if constexpr (D <= 512) {
    if (G == 4) return bf16 ? ffpa::launch_dec_bwd<D, true, 4> : ffpa::launch_dec_bwd<D, false, 4>;
  }
  return nullptr;
}

DecBwdLauncher dec_bwd_launcher(int D, int bf16, int G) {
  switch (D) {
#define FFPA_CASE(DD) \
  case DD:            \
    return dec_bwd_pick<DD>(bf16, G);
    FFPA_CASE(64) FFPA_CASE(128) FFPA_CASE(192) FFPA_CASE(256) FFPA_CASE(320) FFPA_CASE(384)
    FFPA_CASE(448) FFPA_CASE(512) FFPA_CASE(576) FFPA_CASE(640) FFPA_CASE(704) FFPA_CASE(768)
    FFPA_CASE(832) FFPA_CASE(896) FFPA_CASE(960) FFPA_CASE(1024)
#undef FFPA_CASE
    default:
      return nullptr;
  }
}

// Whether the decode backward serves this shape (the size query cannot know
// about dropout; a call with dropout takes the other kernels).
bool dec_bwd_built(int Nq, int Hq, int Hkv, int Nkv, int D) {
  if (Nq != 1 || Hkv < 1 || Hq % Hkv != 0 || Nkv < 1) return false;
  return dec_bwd_launcher(D, 0, Hq / Hkv) != nullptr;
}

int64_t bwd_nq_pad(int Nq) { return ((int64_t)Nq + ffpa::kBwdPad - 1) / ffpa::kBwdPad * ffpa::kBwdPad; }

// Checks shared by forward and backward; returns FFPA_OK or an error code.
int check_common(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, const void* mask,
                 int mask_rows, int accum_dtype, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1)
    return fail(FFPA_ERR_INVALID_ARG, "sizes B, Hq, Hkv, Nq, Nkv, D must all be >= 1");
  if (Hq % Hkv != 0) return fail(FFPA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (causal != 0 && causal != 1) return fail(FFPA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (mask != nullptr && mask_rows != 1 && mask_rows != Nq)
    return fail(FFPA_ERR_INVALID_ARG, "mask_rows must be 1 or Nq");
  if (dtype != FFPA_F16 && dtype != FFPA_BF16) return fail(FFPA_ERR_UNSUPPORTED, "dtype must be FFPA_F16 or FFPA_BF16");
  if (accum_dtype != FFPA_ACC_F32 && accum_dtype != FFPA_ACC_F16)
    return fail(FFPA_ERR_UNSUPPORTED, "accum_dtype must be FFPA_ACC_F32 or FFPA_ACC_F16");
  if (D % 32 != 0 || D > FFPA_MAX_HEAD_DIM)
    return fail(FFPA_ERR_UNSUPPORTED, "D must be a multiple of 32 and at most 1024");
  // byte offsets inside one (b, h) slice, one tile past its end included, fit 32 bits
  if ((int64_t)(Nq + 128) * D >= (int64_t(1) << 31) || (int64_t)(Nkv + 128) * D >= (int64_t(1) << 31))
    return fail(FFPA_ERR_UNSUPPORTED, "(N + 128) * D must be below 2^31");
  if ((int64_t)B * Hq >= (int64_t(1) << 31))
    return fail(FFPA_ERR_UNSUPPORTED, "B * Hq too large");
  return FFPA_OK;
}

}  // namespace

extern "C" {

int ffpa_version(void) { return 100; }

const char* ffpa_last_error(void) { return g_err.c_str(); }

size_t ffpa_attn_fwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype) {
  (void)dtype;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1) return 0;
  if (Nq == 1) {
    // decode: per key range, o (D fp32) and a log-sum-exp (fp32); the causal
    // variant uses fewer ranges, so the non-causal count bounds both
    const size_t s = (size_t)ffpa::dec_splits(B, Hq, Nkv);
    return (size_t)B * Hq * s * ((size_t)D + 1) * sizeof(float);
  }
  // the transposed copy of V the attention kernels read (always above
  // D = 512; up to 512 when the problem repays the pass)
  if (D % 64 == 0 && (D > 512 || ffpa::fwd_use_vt(Hq, Hkv, Nq))) return ffpa::fwd_vt_bytes(B, Hkv, Nkv, D);
  return 0;
}

}  // extern "C"

namespace {

// Dropout parameters from a probability: threshold t = round(256 p) in
// float32 (an element is kept when its generator byte is >= t), the scale of
// a kept element 256 / (256 - t). p must lie in [0, 1); t = 0 means none.
int drop_params(float p, uint64_t seed, ffpa::DropParams* d) {
  if (!(p >= 0.f && p < 1.f)) return fail(FFPA_ERR_INVALID_ARG, "dropout_p must lie in [0, 1)");
  const float t = std::min(std::floor(256.f * p + 0.5f), 255.f);
  d->t = (uint32_t)t;
  d->seed_lo = (uint32_t)seed;
  d->seed_hi = (uint32_t)(seed >> 32);
  d->scale = d->t ? 256.f / (256.f - t) : 1.f;
  return FFPA_OK;
}

// Checks of ffpa_attn_fwd's arguments that come before the workspace.
int fwd_check_args(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                   int Hkv, int Nq, int Nkv, int D, float scale, int causal, const void* mask,
                   int mask_rows, int accum_dtype, int dtype) {
  if (!q || !k || !v || !o) return fail(FFPA_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  const int st = check_common(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(mask))
    return fail(FFPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!(scale == scale)) return fail(FFPA_ERR_INVALID_ARG, "scale is NaN");
  return FFPA_OK;
}

// Forward variants: the tile shapes and staging layouts a problem can run
// with (ffpa_attn_fwd_variant, ffpa_attn_fwd_tune). 0 = the default choice.
//   Nq > 1, D <= 512: 1 = V staged as is, 2 = V from its transposed copy;
//   Nq > 1, D > 512:  WideShape (1 = fp32 accumulator, 64 rows; 2 = fp16
//                     accumulator, a wave holds all of D, 128 rows, D <= 768,
//                     the prefill kernel at 576 and 640; 3 = fp16
//                     accumulator, a wave pair splits D, 64 rows);
//   Nq = 1:           1, 2, 3 = the default number of key ranges per head
//                     divided by 1, 2, 4.
constexpr int kMaxVariant = 3;

// The variant 0 stands for, for this problem.
int fwd_default_variant(int Hq, int Hkv, int Nq, int D, int accum_dtype, bool dropout) {
  if (Nq == 1) return 1;
  if (D > 512) return (dropout || accum_dtype != FFPA_ACC_F16) ? kWideF32 : (D <= 768 ? kWide16One : kWide16Two);
  return ffpa::fwd_use_vt(Hq, Hkv, Nq) ? 2 : 1;
}

// Whether `variant` (after 0 is resolved) exists for this problem: the fp16-
// accumulator shapes only where fp16 accumulation was asked for (fp32 is the
// more accurate one), and not with dropout.
bool fwd_variant_ok(int Nq, int D, int accum_dtype, bool dropout, int variant) {
  if (variant < 1 || variant > kMaxVariant) return false;
  if (Nq == 1) return true;
  if (D > 512) {
    if (variant == kWideF32) return true;
    if (dropout || accum_dtype != FFPA_ACC_F16) return false;
    return variant == kWide16Two || D <= 768;
  }
  return variant <= 2;
}

// Decode key ranges per head under `variant`.
int dec_splits_for(int B, int Hq, int kv_end, int variant) {
  const int s = ffpa::dec_splits(B, Hq, kv_end);
  const int div = variant == 3 ? 4 : variant == 2 ? 2 : 1;
  return std::max(1, s / div);
}

// Workspace bytes of a resolved variant.
size_t fwd_variant_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int variant) {
  if (Nq == 1)
    return (size_t)B * Hq * dec_splits_for(B, Hq, dec_kv_end(Nkv, causal), variant) * ((size_t)D + 1) * sizeof(float);
  if (D > 512 || variant == 2) return ffpa::fwd_vt_bytes(B, Hkv, Nkv, D);
  return 0;
}

// The forward after its argument checks, as `variant` (0 = default).
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nkv, int D, float scale, int causal, const void* mask,
             int mask_rows, int accum_dtype, int dtype, void* workspace, size_t workspace_bytes,
             int variant, void* stream, const ffpa::DropParams& drop = ffpa::DropParams{}) {
  const bool dropout = drop.t != 0;
  if (dropout && accum_dtype != FFPA_ACC_F32)
    return fail(FFPA_ERR_UNSUPPORTED, "dropout is built with the fp32 accumulator (FFPA_ACC_F32)");
  if (variant == 0) variant = fwd_default_variant(Hq, Hkv, Nq, D, accum_dtype, dropout);
  if (!fwd_variant_ok(Nq, D, accum_dtype, dropout, variant))
    return fail(FFPA_ERR_INVALID_ARG, "variant " + std::to_string(variant) + " does not exist for this problem");
  if (!aligned16(workspace)) return fail(FFPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t need = fwd_variant_bytes(B, Hq, Hkv, Nq, Nkv, D, causal, variant);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr))
    return fail(FFPA_ERR_WORKSPACE, "workspace smaller than this path needs (ffpa_attn_fwd_workspace_size())");

  if (Nq == 1) {
    // one query row per head: split-KV decode kernels
    DecLauncher launch = dec_launcher(D, dtype == FFPA_BF16);
    if (launch == nullptr) return fail(FFPA_ERR_UNSUPPORTED, "this head dimension is not built yet");
    ffpa::DecArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.mask = mask;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nkv = Nkv;
    a.kv_end = dec_kv_end(Nkv, causal);
    a.splits = dec_splits_for(B, Hq, a.kv_end, variant);
    a.keys_per_split = ffpa::dec_keys_per_split(a.kv_end, a.splits);
    a.scale_log2 = scale * ffpa::kLog2e;
    const int64_t waves = (int64_t)B * Hq * a.splits;
    if (waves >= (int64_t(1) << 31)) return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
    a.n_waves = (int)waves;
    a.part_o = (float*)workspace;
    a.part_lse = (float*)workspace + (size_t)waves * D;
    a.drop = drop;
    hipError_t e = launch(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return FFPA_OK;
  }

  // 576 and 640 with the fp16 accumulator, one part of D per wave: the
  // prefill kernel (64-key tiles, V^T staged) serves that tile shape
  const bool prefill_wide = (D == 576 || D == 640) && variant == kWide16One && !dropout &&
                            accum_dtype == FFPA_ACC_F16;
  if (D > 512 && !prefill_wide) {
    // head dimensions above 512
    int rows = 64;
    WideLauncher launch = wide_launcher(D, dtype == FFPA_BF16, variant, dropout, &rows);
    if (launch == nullptr)
      return fail(FFPA_ERR_UNSUPPORTED, "for Nq > 1, D above 512 must be a multiple of 64");
    ffpa::FwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.mask = mask;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv;
    a.mask_rows = mask ? mask_rows : 0;
    a.mask_stride = (mask && mask_rows > 1) ? Nkv : 0;
    a.bias_lds = 0;
    a.causal = causal;
    a.scale_log2 = scale * ffpa::kLog2e;
    a.n_qtiles = (Nq + rows - 1) / rows;
    const int64_t total = (int64_t)B * Hq * a.n_qtiles;
    if (total >= (int64_t(1) << 31)) return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
    a.total_wg = (int)total;
    a.vt = workspace;
    a.nkv_pad = ffpa::fwd_nkv_pad(Nkv);
    a.drop = drop;
    if (!ffpa::fwd_vt_grid_ok(B * Hkv, Nkv, D)) return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
    const hipError_t e = launch(a, (hipStream_t)stream);  // V^T pass, then the kernel
    if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return FFPA_OK;
  }

  size_t ring = 0;
  const bool vt = variant == 2;
  FwdLauncher launch = fwd_launcher(D, dtype == FFPA_BF16, accum_dtype == FFPA_ACC_F16, vt, dropout, &ring);
  if (launch == nullptr) return fail(FFPA_ERR_UNSUPPORTED, "this head dimension is not built yet");
  // the restart flags: fp32 accumulation only
  size_t lds = ring + (accum_dtype == FFPA_ACC_F16 ? 0 : ffpa::kFwdFlagBytes);
  // a key bias is staged in LDS when it fits beside the tiles; otherwise the
  // kernel reads it (like a per-query mask) from global memory
  const bool bias_lds = mask != nullptr && mask_rows == 1 &&
                        lds + (size_t)ffpa::fwd_bias_bytes(Nkv) <= kLdsLimit;
  if (bias_lds) lds += (size_t)ffpa::fwd_bias_bytes(Nkv);

  ffpa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.mask = mask;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv;
  a.mask_rows = mask ? mask_rows : 0;
  a.mask_stride = (mask && mask_rows > 1) ? Nkv : 0;
  a.bias_lds = bias_lds ? 1 : 0;
  a.causal = causal;
  a.scale_log2 = scale * ffpa::kLog2e;
  a.n_qtiles = (Nq + ffpa::kFwdRows - 1) / ffpa::kFwdRows;
  const int64_t total = (int64_t)B * Hq * a.n_qtiles;
  if (total >= (int64_t(1) << 31)) return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
  a.total_wg = (int)total;
  a.vt = workspace;
  a.nkv_pad = ffpa::fwd_nkv_pad(Nkv);
  a.drop = drop;
  if (vt && !ffpa::fwd_vt_grid_ok(B * Hkv, Nkv, D)) return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
  const hipError_t e = launch(a, lds, (hipStream_t)stream);  // [V^T pass,] the kernel
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return FFPA_OK;
}

// ---------------------------------------------------------------------------
// Tuned choices: problem key -> variant, filled by ffpa_attn_fwd_tune and read
// by ffpa_attn_fwd (and ffpa_attn_fwd_noalloc) for the rest of the process.
// ---------------------------------------------------------------------------
using TuneKey = std::array<int64_t, 11>;
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tuned;

TuneKey tune_key(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, const void* mask, int mask_rows,
                 int accum_dtype, int dtype) {
  return {B, Hq, Hkv, Nq, Nkv, D, causal, mask ? mask_rows : 0, accum_dtype, dtype, 0};
}

// The tuned variant of this problem if it is recorded and fits the
// workspace given; else 0 (the default).
int tuned_variant(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, const void* mask, int mask_rows,
                  int accum_dtype, int dtype, size_t workspace_bytes) {
  int var = 0;
  {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    const auto it = g_tuned.find(tune_key(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype));
    if (it != g_tuned.end()) var = it->second;
  }
  if (var != 0 && fwd_variant_bytes(B, Hq, Hkv, Nq, Nkv, D, causal, var) > workspace_bytes) var = 0;
  return var;
}

}  // namespace

extern "C" {

int ffpa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                  int Hkv, int Nq, int Nkv, int D, float scale, int causal, const void* mask,
                  int mask_rows, int accum_dtype, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
  g_err.clear();
  const int st = fwd_check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                                accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  const int var = tuned_variant(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype,
                                workspace ? workspace_bytes : 0);
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows, accum_dtype,
                  dtype, workspace, workspace_bytes, var, stream);
}

size_t ffpa_attn_fwd_variant_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype,
                                            int causal, int variant) {
  (void)dtype;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1 || variant < 0 || variant > kMaxVariant) return 0;
  if (variant == 0) return ffpa_attn_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype);
  return fwd_variant_bytes(B, Hq, Hkv, Nq, Nkv, D, causal, variant);
}

int ffpa_attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          int Hkv, int Nq, int Nkv, int D, float scale, int causal, const void* mask,
                          int mask_rows, int accum_dtype, int dtype, int variant, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err.clear();
  const int st = fwd_check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                                accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  if (variant < 0 || variant > kMaxVariant)
    return fail(FFPA_ERR_INVALID_ARG, "variant must be 0 .. " + std::to_string(kMaxVariant));
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows, accum_dtype,
                  dtype, workspace, workspace_bytes, variant, stream);
}

int ffpa_attn_fwd_tune(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                       int Hkv, int Nq, int Nkv, int D, float scale, int causal, const void* mask,
                       int mask_rows, int accum_dtype, int dtype, void* workspace, size_t workspace_bytes,
                       int level, int* chosen, float* ms, void* stream) {
  g_err.clear();
  const int st = fwd_check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                                accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  if (level != 1 && level != 2) return fail(FFPA_ERR_INVALID_ARG, "level must be 1 (fast) or 2 (max)");
  if (!aligned16(workspace)) return fail(FFPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const int warm = level == 1 ? 1 : 3, reps = level == 1 ? 3 : 10;
  const size_t ws_bytes = workspace ? workspace_bytes : 0;
  bool runs[kMaxVariant + 1] = {};
  int n_run = 0;
  for (int var = 1; var <= kMaxVariant; ++var) {
    runs[var] = fwd_variant_ok(Nq, D, accum_dtype, false, var) &&
                fwd_variant_bytes(B, Hq, Hkv, Nq, Nkv, D, causal, var) <= ws_bytes;
    n_run += runs[var];
    if (ms) ms[var - 1] = -1.f;
  }
  if (n_run == 0) return fail(FFPA_ERR_WORKSPACE, "no variant fits the workspace given");
  hipEvent_t ev[2] = {nullptr, nullptr};
  hipError_t e = hipEventCreate(&ev[0]);
  if (e == hipSuccess) e = hipEventCreate(&ev[1]);
  if (e != hipSuccess) {
    for (hipEvent_t x : ev)
      if (x) (void)hipEventDestroy(x);
    return fail(FFPA_ERR_HIP, std::string("hipEventCreate failed: ") + hipGetErrorString(e));
  }
  int best = 0, status = FFPA_OK;
  float best_ms = 0.f;
  for (int var = 1; var <= kMaxVariant && status == FFPA_OK; ++var) {
    float t = -1.f;
    if (runs[var]) {
      for (int i = 0; i < warm + reps && status == FFPA_OK; ++i) {
        if (i == warm && (e = hipEventRecord(ev[0], (hipStream_t)stream)) != hipSuccess) break;
        status = fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows, accum_dtype,
                          dtype, workspace, workspace_bytes, var, stream);
      }
      if (status != FFPA_OK) break;
      if (e == hipSuccess) e = hipEventRecord(ev[1], (hipStream_t)stream);
      if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[0], ev[1]);
      if (e != hipSuccess) break;
      t /= reps;
      if (best == 0 || t < best_ms) {
        best = var;
        best_ms = t;
      }
    }
    if (ms) ms[var - 1] = t;
  }
  for (hipEvent_t x : ev) (void)hipEventDestroy(x);
  if (status != FFPA_OK) return status;
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("timing failed: ") + hipGetErrorString(e));
  {
    std::lock_guard<std::mutex> lock(g_tune_mu);
    g_tuned[tune_key(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype)] = best;
  }
  if (chosen) *chosen = best;
  // o and lse end with the chosen variant's results
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows, accum_dtype, dtype,
                  workspace, workspace_bytes, best, stream);
}

size_t ffpa_attn_fwd_fp8_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || D < 1) return 0;
  return ffpa::f8_workspace_bytes(B, Hq, Hkv, Nq, Nkv, D);
}

int ffpa_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                      int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_err.clear();
  const int st = fwd_check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, nullptr, 0,
                                FFPA_ACC_F32, dtype);
  if (st != FFPA_OK) return st;
  Fp8Launcher launch = fp8_launcher(D, dtype == FFPA_BF16);
  if (launch == nullptr) return fail(FFPA_ERR_UNSUPPORTED, "the fp8 forward is built for D = 128, 192, ..., 512");
  if (!aligned16(workspace)) return fail(FFPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t need = ffpa::f8_workspace_bytes(B, Hq, Hkv, Nq, Nkv, D);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FFPA_ERR_WORKSPACE, "workspace smaller than ffpa_attn_fwd_fp8_workspace_size()");
  ffpa::Fp8Args a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv;
  a.causal = causal;
  a.scale_log2 = scale * ffpa::kLog2e;
  a.nkt = (Nkv + ffpa::kF8Bc - 1) / ffpa::kF8Bc;
  a.n_qtiles = (Nq + ffpa::kF8Rows - 1) / ffpa::kF8Rows;
  const int64_t total = (int64_t)B * Hq * a.n_qtiles;
  constexpr int R = ffpa::kF8AmaxRows;
  const int64_t amax_wg = (int64_t)B * Hq * ((Nq + R - 1) / R) + 2 * (int64_t)B * Hkv * ((Nkv + R - 1) / R);
  const int64_t n16 = ((int64_t)B * Hq * Nq + (int64_t)B * Hkv * Nkv) * (D / 16);
  if (total >= (int64_t(1) << 31) || amax_wg >= (int64_t(1) << 31) || (n16 + 255) / 256 >= (int64_t(1) << 31) ||
      (int64_t)B * Hkv * a.nkt >= (int64_t(1) << 31) || (int64_t)a.nkt * ffpa::kF8Bc * D >= (int64_t(1) << 32))
    return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
  a.total_wg = (int)total;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = (char*)workspace;
  a.amax = (float*)w;
  w += ffpa::f8_amax_bytes(B, Hq);
  a.q8 = (uint8_t*)w;
  w += up((size_t)B * Hq * Nq * D);
  a.k8 = (uint8_t*)w;
  w += up((size_t)B * Hkv * Nkv * D);
  a.vt8 = (uint8_t*)w;
  const hipError_t e = launch(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return FFPA_OK;
}

void ffpa_attn_tune_reset(void) {
  std::lock_guard<std::mutex> lock(g_tune_mu);
  g_tuned.clear();
}

int ffpa_attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                          int Hkv, int Nq, int Nkv, int D, float scale, int causal, const void* mask,
                          int mask_rows, int accum_dtype, int dtype, float dropout_p, uint64_t seed,
                          void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  const int st = fwd_check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                                accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  ffpa::DropParams drop{};
  const int dst = drop_params(dropout_p, seed, &drop);
  if (dst != FFPA_OK) return dst;
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows, accum_dtype,
                  dtype, workspace, workspace_bytes, 0, stream, drop);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch of ffpa_attn_fwd_noalloc: one array in each GPU's memory, from the
// library's load until the process ends. In host code `scratch` is only a
// stand-in symbol: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and host code uses that address
// (never the array's name) wherever it needs the memory.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the device that runs `stream` (the
// current device for the null stream), looked up on the first call there.
int scratch_address(void* stream, void** out) {
  int dev = -1, cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e == hipSuccess) e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("no device for the stream: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FFPA_ERR_UNSUPPORTED, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(FFPA_ERR_HIP, std::string("hipSetDevice failed: ") + hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    const hipError_t back = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || ptr == nullptr)
      return fail(FFPA_ERR_HIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    if (back != hipSuccess)
      return fail(FFPA_ERR_HIP, std::string("hipSetDevice failed: ") + hipGetErrorString(back));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FFPA_OK;
}

}  // namespace

extern "C" {

int ffpa_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                          const void* mask, int mask_rows, int accum_dtype, int dtype, void* stream) {
  g_err.clear();
  const int st = fwd_check_args(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                                accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  const size_t need = ffpa_attn_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype);
  if (need <= kNoAllocScratchBytes) {
    void* ws = nullptr;
    const int sa = scratch_address(stream, &ws);
    if (sa != FFPA_OK) return sa;
    // the variant ffpa_attn_fwd would take with this much workspace
    const int var = tuned_variant(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype,
                                  kNoAllocScratchBytes);
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows, accum_dtype,
                    dtype, ws, kNoAllocScratchBytes, var, stream);
  }
  if (Nq > 1 && D <= 512)  // V staged as is: no scratch at all
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows, accum_dtype,
                    dtype, nullptr, 0, 1, stream);
  return fail(FFPA_ERR_WORKSPACE, "these sizes need " + std::to_string(need) +
                                      " bytes of scratch; ffpa_attn_fwd_noalloc holds " +
                                      std::to_string(kNoAllocScratchBytes));
}

size_t ffpa_attn_bwd_workspace_size_min(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype) {
  (void)Hkv; (void)Nkv; (void)D; (void)dtype;
  if (B < 1 || Hq < 1 || Nq < 1) return 0;
  // delta and lse * log2(e) per query row, rows padded to a multiple of 64
  return 2 * (size_t)B * Hq * (size_t)bwd_nq_pad(Nq) * sizeof(float);
}

// bytes of the stored-dS path's K^T copy and of the dS blocks of one kv
// head's query heads (after the row data)
static size_t bwd_kt_bytes(int B, int Hkv, int Nkv, int D) {
  return (size_t)B * Hkv * D * (size_t)ffpa::fwd_nkv_pad(Nkv) * 2;
}
static size_t bwd_ds_bytes_kvhead(int Hq, int Hkv, int Nq, int Nkv) {
  return (size_t)(Hq / Hkv) * (size_t)((Nq + 31) / 32) * (size_t)((Nkv + 31) / 32) * 2048;
}

// dS budget of the size query: the dK/dV and dQ passes run over chunks of kv
// heads whose dS fits it (at least one kv head's group per chunk), and of
// at least as many kv heads as give a chunk's dQ pass kBwdDqMinWg workgroups
// (two per CU): with fewer, the causal rows' very different lengths leave
// most CUs idle behind the longest (16K causal: 641 -> 722 TFLOP/s).
constexpr size_t kBwdDsBudget = size_t(1) << 30;
constexpr int64_t kBwdDqMinWg = 512;

static int bwd_default_chunk(int B, int Hq, int Hkv, int Nq, int Nkv, int D) {
  const size_t per = bwd_ds_bytes_kvhead(Hq, Hkv, Nq, Nkv);
  const int64_t nkv = (int64_t)B * Hkv;
  const int dq_rows = D <= 512 ? 128 : 64;  // query rows per dQ workgroup
  const int64_t dq_wg_per_kv = (int64_t)(Hq / Hkv) * ((Nq + dq_rows - 1) / dq_rows);
  const int64_t fit = std::max<int64_t>((int64_t)(kBwdDsBudget / per),
                                        (kBwdDqMinWg + dq_wg_per_kv - 1) / dq_wg_per_kv);
  // equal chunks: the fewest that respect the budget, then the chunk size
  // that spreads the heads evenly over them
  const int64_t chunks = (nkv + std::max<int64_t>(fit, 1) - 1) / std::max<int64_t>(fit, 1);
  return (int)((nkv + chunks - 1) / chunks);
}

size_t ffpa_attn_bwd_workspace_size_stored(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype) {
  const size_t base = ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, dtype);
  if (base == 0 || Hkv < 1 || Nkv < 1 || D < 1 || Hq % Hkv != 0) return base;
  const int chunk = bwd_default_chunk(B, Hq, Hkv, Nq, Nkv, D);
  return base + bwd_kt_bytes(B, Hkv, Nkv, D) + (size_t)chunk * bwd_ds_bytes_kvhead(Hq, Hkv, Nq, Nkv);
}

size_t ffpa_attn_bwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype) {
  const size_t base = ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, dtype);
  if (base == 0) return 0;  // no valid problem (B, Hq or Nq below 1)
  // one query row: the decode backward (dQ partials of each key range)
  if (dec_bwd_built(Nq, Hq, Hkv, Nkv, D)) return std::max(base, ffpa::dec_bwd_bytes(B, Hq, Hkv, Nkv, D));
  // up to 64 query rows a head's dQ is one workgroup that reads K and V once:
  // cheaper than the K transpose the stored-dS path needs
  if (Nq <= 64) return base;
  return ffpa_attn_bwd_workspace_size_stored(B, Hq, Hkv, Nq, Nkv, D, dtype);
}

}  // extern "C"

namespace {

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
             int Nkv, int D, float scale, int causal, const void* mask, int mask_rows,
             int accum_dtype, int dtype, void* workspace, size_t workspace_bytes, void* stream,
             bool with_drop, float dropout_p, uint64_t seed) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(FFPA_ERR_INVALID_ARG, "q, k, v, o, dout, lse, dq, dk and dv must be non-null");
  int st = check_common(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  if (accum_dtype != FFPA_ACC_F32)
    return fail(FFPA_ERR_UNSUPPORTED, "the backward accumulates in fp32 only (FFPA_ACC_F32)");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(mask) ||
      !aligned16(workspace))
    return fail(FFPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  ffpa::DropParams drop{};
  if (with_drop) {
    const int dst = drop_params(dropout_p, seed, &drop);
    if (dst != FFPA_OK) return dst;
  }
  const size_t need = ffpa_attn_bwd_workspace_size_min(B, Hq, Hkv, Nq, Nkv, D, dtype);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FFPA_ERR_WORKSPACE, "workspace smaller than ffpa_attn_bwd_workspace_size_min()");
  // room for K^T and the dS of at least one kv head's group: dS is stored by
  // the dK/dV pass and dQ reads it back, over chunks of kv heads that fit
  const size_t kt_b = bwd_kt_bytes(B, Hkv, Nkv, D);
  const size_t ds_per = bwd_ds_bytes_kvhead(Hq, Hkv, Nq, Nkv);
  const size_t room = workspace_bytes > need + kt_b ? workspace_bytes - need - kt_b : 0;
  const bool store_ds = room >= ds_per;
  const int chunk_kv = store_ds ? (int)std::min<size_t>((size_t)B * Hkv, room / ds_per) : 0;
  if (!(scale == scale)) return fail(FFPA_ERR_INVALID_ARG, "scale is NaN");
  BwdLauncher launch = bwd_launcher(D, dtype == FFPA_BF16);
  if (launch == nullptr)
    return fail(FFPA_ERR_UNSUPPORTED, "the backward is built for D = 64, 128, ..., 1024");

  // one query row, no dropout, and room for the dQ partials but not for the
  // stored-dS path: the decode backward (a stream over K and V on the vector
  // ALUs; the dK/dV kernel's 32-row query tiles would be 31/32 empty)
  if (!store_ds && !with_drop && dec_bwd_built(Nq, Hq, Hkv, Nkv, D) &&
      workspace_bytes >= std::max(need, ffpa::dec_bwd_bytes(B, Hq, Hkv, Nkv, D))) {
    DecBwdLauncher dlaunch = dec_bwd_launcher(D, dtype == FFPA_BF16, Hq / Hkv);
    ffpa::DecBwdArgs d{};
    d.q = q; d.k = k; d.v = v; d.o = o; d.dout = dout; d.lse = lse; d.mask = mask;
    d.dq = dq; d.dk = dk; d.dv = dv;
    d.part_dq = (float*)workspace;
    d.B = B; d.Hq = Hq; d.Hkv = Hkv; d.Nkv = Nkv;
    d.kv_end = dec_kv_end(Nkv, causal);
    d.splits = ffpa::dec_bwd_splits(B, Hkv, Nkv);
    d.keys_per_split = ffpa::dec_keys_per_split(Nkv, d.splits);
    d.scale = scale;
    d.scale_log2 = scale * ffpa::kLog2e;
    const int64_t waves = (int64_t)B * Hkv * d.splits;
    if (waves >= (int64_t(1) << 31) - 3 || (int64_t)B * Hq >= (int64_t(1) << 31) - 3)
      return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
    d.n_waves = (int)waves;
    const hipError_t e = dlaunch(d, (hipStream_t)stream);
    if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return FFPA_OK;
  }

  ffpa::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.mask = mask;
  a.mask_rows = mask ? mask_rows : 0;
  const int64_t nq_pad = bwd_nq_pad(Nq);
  a.delta = (float*)workspace;
  a.lse2 = (float*)workspace + (size_t)B * Hq * nq_pad;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv;
  a.nq_pad = (int)nq_pad;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * ffpa::kLog2e;
  a.drop = drop;
  a.bh0 = 0;
  const int rows = ffpa::bwd_rows_per_wg(D);  // keys per dK/dV workgroup, queries per dQ one
  const int64_t wg_dkdv = (int64_t)B * Hkv * ((Nkv + rows - 1) / rows);
  const int64_t wg_dq = (int64_t)B * Hq * ((Nq + rows - 1) / rows);
  if (wg_dkdv >= (int64_t(1) << 31) || wg_dq >= (int64_t(1) << 31) ||
      (int64_t)B * Hq * nq_pad / 4 >= (int64_t(1) << 31))
    return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
  a.wg_dkdv = (int)wg_dkdv;
  a.wg_dq = (int)wg_dq;
  if (store_ds) {
    const int rq = ffpa::bwd_dq_ds_rows(D);
    const int64_t wg_dq_ds = (int64_t)B * Hq * ((Nq + rq - 1) / rq);
    if (wg_dq_ds >= (int64_t(1) << 31) || !ffpa::fwd_vt_grid_ok(B * Hkv, Nkv, D))
      return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
    a.wg_dq_ds = (int)wg_dq_ds;
    a.nqt = (Nq + 31) / 32;
    a.nkt = (Nkv + 31) / 32;
    a.nkv_pad = ffpa::fwd_nkv_pad(Nkv);
    a.kt = (char*)workspace + need;
    a.ds = (char*)a.kt + kt_b;
  }
  const hipError_t e = launch(a, chunk_kv, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return FFPA_OK;
}

}  // namespace

extern "C" {

int ffpa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                  int Nkv, int D, float scale, int causal, const void* mask, int mask_rows,
                  int accum_dtype, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                  accum_dtype, dtype, workspace, workspace_bytes, stream, false, 0.f, 0);
}

int ffpa_attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                          int Nkv, int D, float scale, int causal, const void* mask, int mask_rows,
                          int accum_dtype, int dtype, float dropout_p, uint64_t seed, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_err.clear();
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, scale, causal, mask, mask_rows,
                  accum_dtype, dtype, workspace, workspace_bytes, stream, true, dropout_p, seed);
}

}  // extern "C"
