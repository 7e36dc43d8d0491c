// Instances of the wide forward kernel (D split across wave pairs) for head dimension 640.
#include "fwd_wide.hpp"

namespace ffpa {
template hipError_t launch_fwd_wide<640, false>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide<640, true>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide<640, false, true>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide<640, true, true>(const FwdArgs&, hipStream_t);
}  // namespace ffpa
