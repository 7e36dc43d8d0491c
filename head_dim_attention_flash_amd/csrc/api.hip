// C ABI of libffpa_attn: argument validation, kernel selection and launch.
// The operation and its conventions are documented in include/ffpa_attn.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "ffpa_attn.h"
#include "fwd_prefill.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

constexpr size_t kLdsLimit = 160 * 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

using FwdLauncher = hipError_t (*)(const ffpa::FwdArgs&, size_t, hipStream_t);

template <int D>
FwdLauncher pick_fwd(int bf16, int acc16) {
  if (bf16) return acc16 ? ffpa::launch_fwd_prefill<D, true, true> : ffpa::launch_fwd_prefill<D, true, false>;
  return acc16 ? ffpa::launch_fwd_prefill<D, false, true> : ffpa::launch_fwd_prefill<D, false, false>;
}

FwdLauncher fwd_launcher(int D, int bf16, int acc16, size_t* ring_bytes) {
  switch (D) {
#define FFPA_CASE(DD)                             \
  case DD:                                        \
    *ring_bytes = ffpa::fwd_ring_bytes<DD>();     \
    return pick_fwd<DD>(bf16, acc16);
    FFPA_CASE(64)
    FFPA_CASE(128)
    FFPA_CASE(192)
    FFPA_CASE(256)
    FFPA_CASE(320)
    FFPA_CASE(384)
    FFPA_CASE(448)
    FFPA_CASE(512)
#undef FFPA_CASE
    default:
      return nullptr;
  }
}

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
  // element counts must index with 32-bit row offsets inside one (b, h) slice
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
  (void)B; (void)Hq; (void)Hkv; (void)Nq; (void)Nkv; (void)D; (void)dtype;
  return 0;
}

int ffpa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                  int Hkv, int Nq, int Nkv, int D, float scale, int causal, const void* mask,
                  int mask_rows, int accum_dtype, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream) {
  g_err.clear();
  if (!q || !k || !v || !o) return fail(FFPA_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  int st = check_common(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(mask))
    return fail(FFPA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  const size_t need = ffpa_attn_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, D, dtype);
  if (workspace_bytes < need || (need > 0 && workspace == nullptr))
    return fail(FFPA_ERR_WORKSPACE, "workspace smaller than ffpa_attn_fwd_workspace_size()");
  if (!(scale == scale)) return fail(FFPA_ERR_INVALID_ARG, "scale is NaN");

  size_t ring = 0;
  FwdLauncher launch = fwd_launcher(D, dtype == FFPA_BF16, accum_dtype == FFPA_ACC_F16, &ring);
  if (launch == nullptr) return fail(FFPA_ERR_UNSUPPORTED, "this head dimension is not built yet");
  size_t lds = ring + ffpa::kFwdFlagBytes;
  if (mask != nullptr) {
    if (mask_rows != 1)
      return fail(FFPA_ERR_UNSUPPORTED, "per-query masks [Nq, Nkv] are not supported yet");
    lds += (size_t)ffpa::fwd_bias_bytes(Nkv);
    if (lds > kLdsLimit)
      return fail(FFPA_ERR_UNSUPPORTED, "key bias does not fit in LDS beside the K/V tiles");
  }

  ffpa::FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.mask = mask;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv;
  a.mask_rows = mask ? 1 : 0;
  a.causal = causal;
  a.scale_log2 = scale * ffpa::kLog2e;
  a.n_qtiles = (Nq + ffpa::kFwdRows - 1) / ffpa::kFwdRows;
  const int64_t total = (int64_t)B * Hq * a.n_qtiles;
  if (total >= (int64_t(1) << 31)) return fail(FFPA_ERR_UNSUPPORTED, "grid too large");
  a.total_wg = (int)total;
  hipError_t e = launch(a, lds, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FFPA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  (void)workspace;
  return FFPA_OK;
}

size_t ffpa_attn_bwd_workspace_size(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int dtype) {
  (void)Hkv; (void)Nkv; (void)D; (void)dtype;
  return (size_t)B * Hq * Nq * sizeof(float);
}

int ffpa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                  int Nkv, int D, float scale, int causal, const void* mask, int mask_rows,
                  int accum_dtype, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(FFPA_ERR_INVALID_ARG, "q, k, v, o, dout, lse, dq, dk and dv must be non-null");
  int st = check_common(B, Hq, Hkv, Nq, Nkv, D, causal, mask, mask_rows, accum_dtype, dtype);
  if (st != FFPA_OK) return st;
  if (accum_dtype != FFPA_ACC_F32)
    return fail(FFPA_ERR_UNSUPPORTED, "the backward accumulates in fp32 only (FFPA_ACC_F32)");
  (void)scale; (void)workspace; (void)workspace_bytes; (void)stream;
  return fail(FFPA_ERR_UNSUPPORTED, "backward kernels are not built yet");
}

}  // extern "C"
