// Instances of the wide forward kernel with the fp16 output accumulator for head dimension 896.
#include "fwd_wide16.hpp"

namespace ffpa {
template hipError_t launch_fwd_wide16<896, false>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide16<896, true>(const FwdArgs&, hipStream_t);
}  // namespace ffpa
