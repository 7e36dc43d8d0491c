// Instances of the wide forward kernel (D split across wave pairs) for head dimension 832.
#include "fwd_wide.hpp"

namespace ffpa {
template hipError_t launch_fwd_wide<832, false>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide<832, true>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide<832, false, true>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide<832, true, true>(const FwdArgs&, hipStream_t);
}  // namespace ffpa
