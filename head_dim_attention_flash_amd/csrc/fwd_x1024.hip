// Instances of the wide forward kernel with the fp16 output accumulator for head dimension 1024.
#include "fwd_wide16.hpp"

namespace ffpa {
template hipError_t launch_fwd_wide16<1024, false>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide16<1024, true>(const FwdArgs&, hipStream_t);
}  // namespace ffpa
