// Backward kernels of the softmax_1 variant (instantiations of bwd_kernel.h).
#include "bwd_kernel.h"

namespace sigattn {

template <int D>
static hipError_t launch_part(const AttnParams &p, hipStream_t stream, int part) {
    if (part == 0) return launch_dkdv_d<D, kSoftmax1>(p, stream);
    if (part == 1) return launch_dq_d<D, kSoftmax1>(p, stream);
    return launch_bwd_d<D, kSoftmax1>(p, stream);
}

hipError_t launch_bwd_softmax1(const AttnParams &p, hipStream_t stream, int part) {
    return p.d == 64 ? launch_part<64>(p, stream, part) : launch_part<128>(p, stream, part);
}

}  // namespace sigattn
