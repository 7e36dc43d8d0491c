// Instances of the forward prefill kernel for head dimension 64.
#include "fwd_prefill.hpp"

namespace ffpa {
template hipError_t launch_fwd_prefill<64, false, false>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<64, true, false>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<64, false, true>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<64, true, true>(const FwdArgs&, size_t, hipStream_t);
}  // namespace ffpa
