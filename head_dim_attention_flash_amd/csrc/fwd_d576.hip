// Instances of the forward prefill kernel for head dimension 576: the fp16
// output accumulator with V staged from its transposed copy only.
#include "fwd_prefill.hpp"

namespace ffpa {
template hipError_t launch_fwd_prefill<576, false, true, true>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<576, true, true, true>(const FwdArgs&, size_t, hipStream_t);
}  // namespace ffpa
