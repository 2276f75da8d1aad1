// Forward kernels of the sigmoid variant (instantiations of fwd_kernel.h).
#include "fwd_kernel.h"

namespace sigattn {

hipError_t launch_fwd_sigmoid(const AttnParams &p, hipStream_t stream) {
    return p.d == 64 ? launch_fwd_d<64, kSigmoid>(p, stream)
                     : launch_fwd_d<128, kSigmoid>(p, stream);
}

}  // namespace sigattn
