// Instances of the backward kernels for head dimension 1024.
#include "bwd.hpp"

namespace ffpa {
template hipError_t launch_bwd<1024, false>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd<1024, true>(const BwdArgs&, int, hipStream_t);
}  // namespace ffpa
