// Instances of the fp8 forward (pre-pass and attention kernel) for every
// head dimension it is built for.
#include "fwd_fp8.hpp"

namespace ffpa {
#define FFPA_INST(DD)                                                           \
  template hipError_t launch_fwd_fp8<DD, false>(const Fp8Args&, hipStream_t); \
  template hipError_t launch_fwd_fp8<DD, true>(const Fp8Args&, hipStream_t);
FFPA_INST(128) FFPA_INST(192) FFPA_INST(256) FFPA_INST(320) FFPA_INST(384) FFPA_INST(448) FFPA_INST(512)
#undef FFPA_INST
}  // namespace ffpa
