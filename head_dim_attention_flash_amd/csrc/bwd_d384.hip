// Instances of the backward kernels for head dimension 384.
#include "bwd.hpp"

namespace ffpa {
template hipError_t launch_bwd<384, false>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd<384, true>(const BwdArgs&, int, hipStream_t);
}  // namespace ffpa
