// Forward kernels of differential attention (instantiations of fwd_kernel.h).
#include "fwd_kernel.h"

namespace sigattn {

// kDiff (d = 64): both maps in one tile loop; kDiffSecond (d = 128, where two
// maps' operands and accumulators do not fit one loop): the second pass of
// the two-pass form.
hipError_t launch_fwd_diff(const AttnParams &p, hipStream_t stream) {
    if (p.variant == kDiffSecond)
        return p.d == 128 ? launch_fwd_d<128, kDiffSecond>(p, stream) : hipErrorInvalidValue;
    return p.d == 64 ? launch_fwd_d<64, kDiff>(p, stream) : hipErrorInvalidValue;
}

}  // namespace sigattn
