// Instances of the forward prefill kernel for head dimension 64.
#include "fwd_prefill.hpp"

namespace ffpa {
#define FFPA_INST(BF, ACC, VT) template hipError_t launch_fwd_prefill<64, BF, ACC, VT>(const FwdArgs&, size_t, hipStream_t);
#define FFPA_INST_DROP(BF, VT) template hipError_t launch_fwd_prefill<64, BF, false, VT, true>(const FwdArgs&, size_t, hipStream_t);
FFPA_INST(false, false, true) FFPA_INST(true, false, true) FFPA_INST(false, true, true) FFPA_INST(true, true, true)
FFPA_INST(false, false, false) FFPA_INST(true, false, false) FFPA_INST(false, true, false) FFPA_INST(true, true, false)
FFPA_INST_DROP(false, true) FFPA_INST_DROP(true, true) FFPA_INST_DROP(false, false) FFPA_INST_DROP(true, false)
#undef FFPA_INST
#undef FFPA_INST_DROP
}  // namespace ffpa
