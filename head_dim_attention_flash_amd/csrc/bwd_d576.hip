// Instances of the backward kernels for head dimension 576.
#include "bwd.hpp"

namespace ffpa {
template hipError_t launch_bwd<576, false>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd<576, true>(const BwdArgs&, int, hipStream_t);
}  // namespace ffpa
