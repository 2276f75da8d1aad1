// Backward kernels of differential attention (instantiations of
// bwd_kernel.h with two softmax maps): both maps' gradients in one pass at
// d = 64, where each work item's two maps fit the register file.
#include "bwd_kernel.h"

namespace sigattn {

hipError_t launch_bwd_diff(const AttnParams &p, hipStream_t stream) {
    if (p.d != 64) return hipErrorInvalidValue;
    return launch_bwd_d<64, kDiff>(p, stream);
}

}  // namespace sigattn
