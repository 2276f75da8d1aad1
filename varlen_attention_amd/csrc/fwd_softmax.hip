// Forward kernels of the softmax and softmax_1 variants (instantiations of fwd_kernel.h).
#include "fwd_kernel.h"

namespace sigattn {

hipError_t launch_fwd_softmax(const AttnParams &p, hipStream_t stream) {
    if (p.variant == kSoftmax)
        return p.d == 64 ? launch_fwd_d<64, kSoftmax>(p, stream)
                         : launch_fwd_d<128, kSoftmax>(p, stream);
    return p.d == 64 ? launch_fwd_d<64, kSoftmax1>(p, stream)
                     : launch_fwd_d<128, kSoftmax1>(p, stream);
}

}  // namespace sigattn
