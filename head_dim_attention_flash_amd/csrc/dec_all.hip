// Instances of the split-KV decode kernels: every head dimension that is a
// multiple of 32 up to 1024, fp16 and bf16.
#include "decode.hpp"

namespace ffpa {
#define FFPA_DEC(D)                                                        \
  template hipError_t launch_decode<D, false>(const DecArgs&, hipStream_t); \
  template hipError_t launch_decode<D, true>(const DecArgs&, hipStream_t);
FFPA_DEC(32) FFPA_DEC(64) FFPA_DEC(96) FFPA_DEC(128) FFPA_DEC(160) FFPA_DEC(192) FFPA_DEC(224)
FFPA_DEC(256) FFPA_DEC(288) FFPA_DEC(320) FFPA_DEC(352) FFPA_DEC(384) FFPA_DEC(416) FFPA_DEC(448)
FFPA_DEC(480) FFPA_DEC(512) FFPA_DEC(544) FFPA_DEC(576) FFPA_DEC(608) FFPA_DEC(640) FFPA_DEC(672)
FFPA_DEC(704) FFPA_DEC(736) FFPA_DEC(768) FFPA_DEC(800) FFPA_DEC(832) FFPA_DEC(864) FFPA_DEC(896)
FFPA_DEC(928) FFPA_DEC(960) FFPA_DEC(992) FFPA_DEC(1024)
#undef FFPA_DEC
}  // namespace ffpa
