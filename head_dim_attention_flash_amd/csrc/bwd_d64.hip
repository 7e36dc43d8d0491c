// Instances of the backward kernels for head dimension 64.
#include "bwd.hpp"

namespace ffpa {
template hipError_t launch_bwd<64, false>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd<64, true>(const BwdArgs&, int, hipStream_t);
}  // namespace ffpa
