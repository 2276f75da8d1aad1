// Forward dispatch: head dimension and variant select the translation unit
// that holds the kernel instantiations (fwd_sigmoid.hip, fwd_softmax.hip,
// fwd_diff.hip); they compile in parallel.
#include "kernels.h"

namespace sigattn {

hipError_t launch_fwd_sigmoid(const AttnParams &p, hipStream_t stream);
hipError_t launch_fwd_softmax(const AttnParams &p, hipStream_t stream);
hipError_t launch_fwd_diff(const AttnParams &p, hipStream_t stream);

hipError_t launch_fwd(const AttnParams &p, hipStream_t stream) {
    if (p.variant == kSigmoid) return launch_fwd_sigmoid(p, stream);
    if (p.variant == kDiff || p.variant == kDiffSecond) return launch_fwd_diff(p, stream);
    return launch_fwd_softmax(p, stream);
}

}  // namespace sigattn
