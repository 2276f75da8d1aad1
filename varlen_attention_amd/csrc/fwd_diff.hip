// Forward kernels of differential attention (instantiations of fwd_kernel.h).
#include "fwd_kernel.h"

namespace sigattn {

hipError_t launch_fwd_diff(const AttnParams &p, hipStream_t stream) {
    return p.d == 64 ? launch_fwd_d<64, kDiff>(p, stream) : launch_fwd_d<128, kDiff>(p, stream);
}

}  // namespace sigattn
