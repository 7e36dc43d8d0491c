// Instances of the backward kernels for head dimension 128.
#include "bwd.hpp"

namespace ffpa {
template hipError_t launch_bwd<128, false>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd<128, true>(const BwdArgs&, int, hipStream_t);
}  // namespace ffpa
