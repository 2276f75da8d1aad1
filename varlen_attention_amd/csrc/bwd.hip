// Backward dispatch: the variant selects the translation unit that holds the
// kernel instantiations (bwd_sigmoid.hip, bwd_softmax.hip, bwd_softmax1.hip,
// bwd_diff.hip); they compile in parallel.
#include "kernels.h"

namespace sigattn {

// part: 0 dK/dV alone, 1 dQ alone, 2 both (one launch when the tile heights agree).
hipError_t launch_bwd_sigmoid(const AttnParams &p, hipStream_t stream, int part);
hipError_t launch_bwd_softmax(const AttnParams &p, hipStream_t stream, int part);
hipError_t launch_bwd_softmax1(const AttnParams &p, hipStream_t stream, int part);
// Differential attention at d = 64, both parts (bwd_diff.hip).
hipError_t launch_bwd_diff(const AttnParams &p, hipStream_t stream);

static hipError_t by_variant(const AttnParams &p, hipStream_t stream, int part) {
    if (p.variant == kDiff) return part == 2 ? launch_bwd_diff(p, stream) : hipErrorInvalidValue;
    if (p.variant == kSigmoid) return launch_bwd_sigmoid(p, stream, part);
    if (p.variant == kSoftmax) return launch_bwd_softmax(p, stream, part);
    return launch_bwd_softmax1(p, stream, part);
}

hipError_t launch_bwd_dkdv(const AttnParams &p, hipStream_t stream) {
    return by_variant(p, stream, 0);
}

hipError_t launch_bwd_dq(const AttnParams &p, hipStream_t stream) {
    return by_variant(p, stream, 1);
}

hipError_t launch_bwd(const AttnParams &p, hipStream_t stream) { return by_variant(p, stream, 2); }

}  // namespace sigattn
