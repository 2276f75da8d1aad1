// Parameter blocks and launchers of the gfx950 kernels.  The host ABI layer
// (api.hip) validates arguments and calls these; each launcher enqueues its
// kernels on the given stream and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sigattn {

// The ABI's variants, plus kDiff: differential attention, two softmax maps
// over one V combined as O1 - lambda O2 (forward only; set by the
// differential entry point).
enum Variant { kSigmoid = 0, kSoftmax = 1, kSoftmax1 = 2, kDiff = 3 };

struct AttnParams {
    const void *q, *k, *v, *dout;   // bf16 [B, H, L, d] (input layout); dout: backward only
    void *o, *dq, *dk, *dv;         // bf16 [B, H, L, d] (output layout)
    float *lse;                     // float [B, H, L] or null
    const void *q2, *k2;            // differential attention: the second map's Q and K
    float *lse2;                    // differential attention: the second map's LSE, or null
    float lambda;                   // differential attention: O = O1 - lambda O2
    void *o1, *o2;                  // differential forward: each map's own output, or null
    float grad_scale;               // backward: every gradient times this (1 normally)
    int accumulate_dv;              // backward: add to dv instead of overwriting it
    const int32_t *seq_lens;        // [B]
    const uint8_t *block_mask;      // [B, Tq, Tk] or null
    const uint8_t *mask;            // [B, L, L] or null
    const int32_t *key_range;       // [B, L, 2] or null (at most one of mask, key_range)
    int64_t sb, sh, sl;             // input strides (elements)
    int64_t osb, osh, osl;          // output strides (elements)
    int B, H, L, d;
    int block_q, block_k, Tq, Tk;   // block-mask geometry
    float scale;
    int bias_mode, variant;
};

hipError_t launch_blockmask(const int32_t *seq_lens, const uint8_t *mask,
                            const int32_t *key_range, int B, int L, int block_q, int block_k,
                            uint8_t *out, hipStream_t stream);
hipError_t launch_fwd(const AttnParams &p, hipStream_t stream);
hipError_t launch_bwd_dkdv(const AttnParams &p, hipStream_t stream);
hipError_t launch_bwd_dq(const AttnParams &p, hipStream_t stream);
// dK, dV and dQ in one launch (two launches when the tile heights differ).
hipError_t launch_bwd(const AttnParams &p, hipStream_t stream);

}  // namespace sigattn
