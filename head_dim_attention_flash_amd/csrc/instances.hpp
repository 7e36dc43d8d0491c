// Explicit instantiation declarations of every kernel launcher the C-ABI
// dispatches to. Each launcher (and the kernels it launches) is instantiated
// in exactly one translation unit (fwd_d*.hip, fwd_w*.hip, fwd_x*.hip,
// bwd_d*.hip, dec_all.hip, fwd_fp8.hip); api.hip includes this header after
// the kernel headers so that it refers to those instances instead of making
// its own copies: one code object per kernel in the library, and a kernel
// header edit cannot leave a stale second copy behind in the dispatcher.
#pragma once

#include "bwd.hpp"
#include "dec_bwd.hpp"
#include "decode.hpp"
#include "fwd_fp8.hpp"
#include "fwd_prefill.hpp"
#include "fwd_wide.hpp"
#include "fwd_wide16.hpp"

namespace ffpa {

#define FFPA_X_PREFILL(D)                                                                              \
  extern template hipError_t launch_fwd_prefill<D, false, false, true>(const FwdArgs&, size_t, hipStream_t); \
  extern template hipError_t launch_fwd_prefill<D, true, false, true>(const FwdArgs&, size_t, hipStream_t);  \
  extern template hipError_t launch_fwd_prefill<D, false, true, true>(const FwdArgs&, size_t, hipStream_t);  \
  extern template hipError_t launch_fwd_prefill<D, true, true, true>(const FwdArgs&, size_t, hipStream_t);   \
  extern template hipError_t launch_fwd_prefill<D, false, false, false>(const FwdArgs&, size_t, hipStream_t); \
  extern template hipError_t launch_fwd_prefill<D, true, false, false>(const FwdArgs&, size_t, hipStream_t);  \
  extern template hipError_t launch_fwd_prefill<D, false, true, false>(const FwdArgs&, size_t, hipStream_t);  \
  extern template hipError_t launch_fwd_prefill<D, true, true, false>(const FwdArgs&, size_t, hipStream_t);   \
  extern template hipError_t launch_fwd_prefill<D, false, false, true, true>(const FwdArgs&, size_t, hipStream_t); \
  extern template hipError_t launch_fwd_prefill<D, true, false, true, true>(const FwdArgs&, size_t, hipStream_t);  \
  extern template hipError_t launch_fwd_prefill<D, false, false, false, true>(const FwdArgs&, size_t, hipStream_t); \
  extern template hipError_t launch_fwd_prefill<D, true, false, false, true>(const FwdArgs&, size_t, hipStream_t);
FFPA_X_PREFILL(64) FFPA_X_PREFILL(128) FFPA_X_PREFILL(192) FFPA_X_PREFILL(256)
FFPA_X_PREFILL(320) FFPA_X_PREFILL(384) FFPA_X_PREFILL(448) FFPA_X_PREFILL(512)
#undef FFPA_X_PREFILL
// 576 and 640: the fp16 accumulator with V^T staged only
#define FFPA_X_PREFILL16(D)                                                                           \
  extern template hipError_t launch_fwd_prefill<D, false, true, true>(const FwdArgs&, size_t, hipStream_t); \
  extern template hipError_t launch_fwd_prefill<D, true, true, true>(const FwdArgs&, size_t, hipStream_t);
FFPA_X_PREFILL16(576) FFPA_X_PREFILL16(640)
#undef FFPA_X_PREFILL16

#define FFPA_X_WIDE(D)                                                                   \
  extern template hipError_t launch_fwd_wide<D, false>(const FwdArgs&, hipStream_t);       \
  extern template hipError_t launch_fwd_wide<D, true>(const FwdArgs&, hipStream_t);        \
  extern template hipError_t launch_fwd_wide<D, false, true>(const FwdArgs&, hipStream_t); \
  extern template hipError_t launch_fwd_wide<D, true, true>(const FwdArgs&, hipStream_t);
#define FFPA_X_WIDE_NH1(D)                                                                 \
  extern template hipError_t launch_fwd_wide16<D, false, 1>(const FwdArgs&, hipStream_t); \
  extern template hipError_t launch_fwd_wide16<D, true, 1>(const FwdArgs&, hipStream_t);
#define FFPA_X_WIDE_NH2(D)                                                                 \
  extern template hipError_t launch_fwd_wide16<D, false, 2>(const FwdArgs&, hipStream_t); \
  extern template hipError_t launch_fwd_wide16<D, true, 2>(const FwdArgs&, hipStream_t);
FFPA_X_WIDE(576) FFPA_X_WIDE(640) FFPA_X_WIDE(704) FFPA_X_WIDE(768)
FFPA_X_WIDE(832) FFPA_X_WIDE(896) FFPA_X_WIDE(960) FFPA_X_WIDE(1024)
// wide16: one wave per 32 rows of all of D at 704 and 768 (at 576 and 640
// that shape is the prefill kernel's); a wave pair per 32 rows at every D
FFPA_X_WIDE_NH1(704) FFPA_X_WIDE_NH1(768)
FFPA_X_WIDE_NH2(576) FFPA_X_WIDE_NH2(640) FFPA_X_WIDE_NH2(704) FFPA_X_WIDE_NH2(768)
FFPA_X_WIDE_NH2(832) FFPA_X_WIDE_NH2(896) FFPA_X_WIDE_NH2(960) FFPA_X_WIDE_NH2(1024)
#undef FFPA_X_WIDE
#undef FFPA_X_WIDE_NH1
#undef FFPA_X_WIDE_NH2

#define FFPA_X_BWD(D)                                                                  \
  extern template hipError_t launch_bwd<D, false>(const BwdArgs&, int, hipStream_t); \
  extern template hipError_t launch_bwd<D, true>(const BwdArgs&, int, hipStream_t);
FFPA_X_BWD(64) FFPA_X_BWD(128) FFPA_X_BWD(192) FFPA_X_BWD(256) FFPA_X_BWD(320) FFPA_X_BWD(384)
FFPA_X_BWD(448) FFPA_X_BWD(512) FFPA_X_BWD(576) FFPA_X_BWD(640) FFPA_X_BWD(704) FFPA_X_BWD(768)
FFPA_X_BWD(832) FFPA_X_BWD(896) FFPA_X_BWD(960) FFPA_X_BWD(1024)
#undef FFPA_X_BWD

#define FFPA_X_DEC(D)                                                                 \
  extern template hipError_t launch_decode<D, false>(const DecArgs&, hipStream_t); \
  extern template hipError_t launch_decode<D, true>(const DecArgs&, hipStream_t);
FFPA_X_DEC(32) FFPA_X_DEC(64) FFPA_X_DEC(96) FFPA_X_DEC(128) FFPA_X_DEC(160) FFPA_X_DEC(192)
FFPA_X_DEC(224) FFPA_X_DEC(256) FFPA_X_DEC(288) FFPA_X_DEC(320) FFPA_X_DEC(352) FFPA_X_DEC(384)
FFPA_X_DEC(416) FFPA_X_DEC(448) FFPA_X_DEC(480) FFPA_X_DEC(512) FFPA_X_DEC(544) FFPA_X_DEC(576)
FFPA_X_DEC(608) FFPA_X_DEC(640) FFPA_X_DEC(672) FFPA_X_DEC(704) FFPA_X_DEC(736) FFPA_X_DEC(768)
FFPA_X_DEC(800) FFPA_X_DEC(832) FFPA_X_DEC(864) FFPA_X_DEC(896) FFPA_X_DEC(928) FFPA_X_DEC(960)
FFPA_X_DEC(992) FFPA_X_DEC(1024)
#undef FFPA_X_DEC

#define FFPA_X_DB(D, G)                                                                          \
  extern template hipError_t launch_dec_bwd<D, false, G>(const DecBwdArgs&, hipStream_t); \
  extern template hipError_t launch_dec_bwd<D, true, G>(const DecBwdArgs&, hipStream_t);
#define FFPA_X_DB_LO(D) FFPA_X_DB(D, 1) FFPA_X_DB(D, 2) FFPA_X_DB(D, 4)
#define FFPA_X_DB_HI(D) FFPA_X_DB(D, 1) FFPA_X_DB(D, 2)
FFPA_X_DB_LO(64) FFPA_X_DB_LO(128) FFPA_X_DB_LO(192) FFPA_X_DB_LO(256)
FFPA_X_DB_LO(320) FFPA_X_DB_LO(384) FFPA_X_DB_LO(448) FFPA_X_DB_LO(512)
FFPA_X_DB_HI(576) FFPA_X_DB_HI(640) FFPA_X_DB_HI(704) FFPA_X_DB_HI(768)
FFPA_X_DB_HI(832) FFPA_X_DB_HI(896) FFPA_X_DB_HI(960) FFPA_X_DB_HI(1024)
#undef FFPA_X_DB_LO
#undef FFPA_X_DB_HI
#undef FFPA_X_DB

#define FFPA_X_FP8(D)                                                                 \
  extern template hipError_t launch_fwd_fp8<D, false>(const Fp8Args&, hipStream_t); \
  extern template hipError_t launch_fwd_fp8<D, true>(const Fp8Args&, hipStream_t);
FFPA_X_FP8(128) FFPA_X_FP8(192) FFPA_X_FP8(256) FFPA_X_FP8(320) FFPA_X_FP8(384) FFPA_X_FP8(448)
FFPA_X_FP8(512)
#undef FFPA_X_FP8

}  // namespace ffpa
