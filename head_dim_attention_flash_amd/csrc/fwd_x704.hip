// Instances of the wide forward kernel with the fp16 output accumulator for head dimension 704.
#include "fwd_wide16.hpp"

namespace ffpa {
template hipError_t launch_fwd_wide16<704, false>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide16<704, true>(const FwdArgs&, hipStream_t);
// the other tile shape (a wave pair splits D, 64 rows per workgroup)
template hipError_t launch_fwd_wide16<704, false, 2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide16<704, true, 2>(const FwdArgs&, hipStream_t);
}  // namespace ffpa
