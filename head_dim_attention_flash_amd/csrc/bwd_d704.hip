// Instances of the backward kernels for head dimension 704.
#include "bwd.hpp"

namespace ffpa {
template hipError_t launch_bwd<704, false>(const BwdArgs&, int, hipStream_t);
template hipError_t launch_bwd<704, true>(const BwdArgs&, int, hipStream_t);
}  // namespace ffpa
