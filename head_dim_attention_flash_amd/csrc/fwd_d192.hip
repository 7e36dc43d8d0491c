// Instances of the forward prefill kernel for head dimension 192.
#include "fwd_prefill.hpp"

namespace ffpa {
template hipError_t launch_fwd_prefill<192, false, false>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<192, true, false>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<192, false, true>(const FwdArgs&, size_t, hipStream_t);
template hipError_t launch_fwd_prefill<192, true, true>(const FwdArgs&, size_t, hipStream_t);
}  // namespace ffpa
