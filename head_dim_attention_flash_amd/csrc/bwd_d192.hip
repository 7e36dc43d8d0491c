// Instances of the backward kernels for head dimension 192.
#include "bwd.hpp"

namespace ffpa {
template hipError_t launch_bwd<192, false>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd<192, true>(const BwdArgs&, int, hipStream_t);
}  // namespace ffpa
