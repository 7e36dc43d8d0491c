// Instances of the forward prefill kernel for head dimension 512.
#include "fwd_prefill.hpp"

namespace ffpa {
template hipError_t launch_fwd_prefill<512, false, false>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<512, true, false>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<512, false, true>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<512, true, true>(const FwdArgs&, size_t, hipStream_t);
}  // namespace ffpa
