// Instances of the wide forward kernel with the fp16 output accumulator for
// head dimension 576: the tile shape where a wave pair splits D (64 rows per
// workgroup). The shape where a wave holds all of D for its 32 rows is the
// prefill kernel's at this D (fwd_d576.hip).
#include "fwd_wide16.hpp"

namespace ffpa {
template hipError_t launch_fwd_wide16<576, false, 2>(const FwdArgs&, hipStream_t);
template hipError_t launch_fwd_wide16<576, true, 2>(const FwdArgs&, hipStream_t);
}  // namespace ffpa
