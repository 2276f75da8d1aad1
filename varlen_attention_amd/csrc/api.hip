// Host side of the C ABI declared in include/sigattn.h: argument validation,
// shape normalisation and dispatch to the kernel launchers.  Nothing here
// allocates memory or synchronises; every call only enqueues work on the
// caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/sigattn.h"
#include "kernels.h"

// Device memory for sigattn_fwd_noalloc's work schedule: one copy per GPU
// (a file-scope device array), held until the process ends.  Host code never
// uses the array's name as an address: scratch_ptr() fetches each device's
// own address once, with hipGetSymbolAddress, and keeps it.
static __device__ __align__(256) uint8_t scratch[SIGATTN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return SIGATTN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool block_size_ok(int b) { return b == 32 || b == 64 || b == 128; }

int launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(SIGATTN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Address of the current device's copy of `scratch` (nullptr and *err set
// on failure), looked up on the device's first use and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

void *scratch_ptr(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Workgroups of the largest launch (the one-launch backward) for B, H, L.
int64_t max_workgroups(int64_t B, int64_t H, int64_t L) {
    return 16 * ((B * H + 7) / 8) * ((L + 127) / 128);
}

// Shared checks of sigattn_fwd / sigattn_bwd; fills the common parameter block.
int check_attention(const sigattn_shape *s, const void *const *inputs, int n_inputs,
                    void *const *outputs, int n_outputs, const int32_t *seq_lens,
                    const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
                    const int32_t *key_range, int32_t bias_mode, int32_t variant,
                    sigattn::AttnParams *p) {
    if (s == nullptr) return fail(SIGATTN_ERR_INVALID_ARG, "shape is NULL");
    if (s->B <= 0 || s->H <= 0 || s->L <= 0)
        return fail(SIGATTN_ERR_INVALID_ARG, "B, H and L must be positive (got %d, %d, %d)",
                    s->B, s->H, s->L);
    if (s->B > 65535 || s->H > 65535)
        return fail(SIGATTN_ERR_UNSUPPORTED, "B and H must be at most 65535");
    // The largest launch, the one-launch backward, has two work items per
    // (batch entry, head) and 128-row tile, the (batch entry, head) pairs
    // rounded up to a multiple of 8 (one share per XCD); its threads
    // (workgroups x 256) must fit HIP's 32-bit grid.  Computed in 64 bits.
    const int64_t bwd_workgroups = max_workgroups(s->B, s->H, s->L);
    if (bwd_workgroups >= SIGATTN_MAX_WORKGROUPS)
        return fail(SIGATTN_ERR_UNSUPPORTED,
                    "B * H * L too large for one launch (%lld workgroups, limit %d)",
                    (long long)bwd_workgroups, SIGATTN_MAX_WORKGROUPS);
    if (s->d != 64 && s->d != 128)
        return fail(SIGATTN_ERR_UNSUPPORTED, "head dim %d not supported (64 or 128)", s->d);
    if (!block_size_ok(s->block_q) || !block_size_ok(s->block_k))
        return fail(SIGATTN_ERR_UNSUPPORTED, "block sizes must be 32, 64 or 128 (got %d, %d)",
                    s->block_q, s->block_k);
    if (bias_mode < SIGATTN_BIAS_NONE || bias_mode > SIGATTN_BIAS_LOG_PADLEN)
        return fail(SIGATTN_ERR_INVALID_ARG, "unknown bias mode %d", bias_mode);
    if (variant < SIGATTN_SIGMOID || variant > SIGATTN_SOFTMAX1)
        return fail(SIGATTN_ERR_INVALID_ARG, "unknown variant %d", variant);
    if (seq_lens == nullptr) return fail(SIGATTN_ERR_INVALID_ARG, "seq_lens is NULL");
    for (int i = 0; i < n_inputs; ++i)
        if (inputs[i] == nullptr) return fail(SIGATTN_ERR_INVALID_ARG, "input %d is NULL", i);
    for (int i = 0; i < n_outputs; ++i)
        if (outputs[i] == nullptr) return fail(SIGATTN_ERR_INVALID_ARG, "output %d is NULL", i);
    if (mask != nullptr && key_range != nullptr)
        return fail(SIGATTN_ERR_INVALID_ARG, "give an element mask or key ranges, not both");
    if ((mask != nullptr || key_range != nullptr) && block_mask == nullptr)
        return fail(SIGATTN_ERR_INVALID_ARG, "an element mask needs its block mask");
    if (schedule != nullptr && block_mask == nullptr)
        return fail(SIGATTN_ERR_INVALID_ARG, "a schedule needs the block mask it was built with");
    if (schedule != nullptr && !aligned16(schedule))
        return fail(SIGATTN_ERR_ALIGNMENT, "schedule is not 16-byte aligned");
    if (key_range != nullptr && (reinterpret_cast<uintptr_t>(key_range) & 7u) != 0)
        return fail(SIGATTN_ERR_ALIGNMENT, "key_range is not 8-byte aligned");
    if (mask != nullptr && s->L > SIGATTN_MAX_MASKED_L)
        return fail(SIGATTN_ERR_UNSUPPORTED, "with an element mask L must be at most %d (got %d)",
                    SIGATTN_MAX_MASKED_L, s->L);
    for (int i = 0; i < n_inputs; ++i)
        if (!aligned16(inputs[i]))
            return fail(SIGATTN_ERR_ALIGNMENT, "input %d is not 16-byte aligned", i);
    for (int i = 0; i < n_outputs; ++i)
        if (!aligned16(outputs[i]))
            return fail(SIGATTN_ERR_ALIGNMENT, "output %d is not 16-byte aligned", i);
    int64_t osb = s->o_stride_b, osh = s->o_stride_h, osl = s->o_stride_l;
    if (osb == 0 && osh == 0 && osl == 0) {
        osb = s->stride_b;
        osh = s->stride_h;
        osl = s->stride_l;
    }
    const int64_t strides[6] = {s->stride_b, s->stride_h, s->stride_l, osb, osh, osl};
    for (int i = 0; i < 6; ++i) {
        if (strides[i] < 0) return fail(SIGATTN_ERR_INVALID_ARG, "negative stride");
        if (strides[i] % 8 != 0)
            return fail(SIGATTN_ERR_ALIGNMENT, "stride %lld is not a multiple of 8 elements",
                        (long long)strides[i]);
    }
    if (s->stride_l < s->d || osl < s->d)
        return fail(SIGATTN_ERR_INVALID_ARG, "row stride smaller than the head dimension");
    if (s->stride_l > SIGATTN_MAX_ROW_STRIDE || osl > SIGATTN_MAX_ROW_STRIDE)
        return fail(SIGATTN_ERR_UNSUPPORTED, "row stride above %d elements",
                    SIGATTN_MAX_ROW_STRIDE);
    p->seq_lens = seq_lens;
    p->block_mask = block_mask;
    p->mask = mask;
    p->key_range = key_range;
    p->sb = s->stride_b;
    p->sh = s->stride_h;
    p->sl = s->stride_l;
    p->osb = osb;
    p->osh = osh;
    p->osl = osl;
    p->B = s->B;
    p->H = s->H;
    p->L = s->L;
    p->d = s->d;
    p->block_q = s->block_q;
    p->block_k = s->block_k;
    p->Tq = (s->L + s->block_q - 1) / s->block_q;
    p->Tk = (s->L + s->block_k - 1) / s->block_k;
    p->scale = s->scale > 0.0f ? s->scale : 1.0f / sqrtf((float)s->d);
    p->grad_scale = 1.0f;
    p->bias_mode = bias_mode;
    p->variant = variant;
    if (schedule != nullptr) {
        const sigattn::ScheduleLayout lay =
            sigattn::schedule_layout(s->B, s->H, s->L, s->block_q, s->block_k, mask != nullptr);
        const uint8_t *base = static_cast<const uint8_t *>(schedule);
        if (mask != nullptr) {  // built with this mask: it holds the mask's bits
            p->mask_bits = reinterpret_cast<const uint32_t *>(base + lay.bits);
            p->bits_w = lay.words_per_row;
        }
        p->items1 = reinterpret_cast<const int4 *>(base + lay.items1);
        p->items2 = reinterpret_cast<const int4 *>(base + lay.items2);
        p->qlist = reinterpret_cast<const uint32_t *>(base + lay.qlists);
        p->klist = reinterpret_cast<const uint32_t *>(base + lay.klists);
        p->qstride = lay.qstride;
        p->kstride = lay.kstride;
    }
    return ok();
}

}  // namespace

extern "C" {

int64_t sigattn_schedule_bytes(int32_t B, int32_t H, int32_t L, int32_t block_q,
                               int32_t block_k, int32_t dense_mask) {
    if (B <= 0 || H <= 0 || L <= 0)
        return fail(SIGATTN_ERR_INVALID_ARG, "B, H and L must be positive");
    if (B > 65535 || H > 65535) return fail(SIGATTN_ERR_UNSUPPORTED, "B and H must be at most 65535");
    if (!block_size_ok(block_q) || !block_size_ok(block_k))
        return fail(SIGATTN_ERR_UNSUPPORTED, "block sizes must be 32, 64 or 128 (got %d, %d)",
                    block_q, block_k);
    if (max_workgroups(B, H, L) >= SIGATTN_MAX_WORKGROUPS)
        return fail(SIGATTN_ERR_UNSUPPORTED, "B * H * L too large for one launch");
    ok();
    return sigattn::schedule_layout(B, H, L, block_q, block_k, dense_mask != 0).bytes;
}

int blockmask_build(const int32_t *seq_lens, const uint8_t *mask, const int32_t *key_range,
                    int32_t B, int32_t H, int32_t L, int32_t block_q, int32_t block_k,
                    uint8_t *block_mask, void *schedule, int64_t schedule_bytes, void *stream) {
    if (seq_lens == nullptr || block_mask == nullptr)
        return fail(SIGATTN_ERR_INVALID_ARG, "seq_lens and block_mask must not be NULL");
    if (B <= 0 || L <= 0) return fail(SIGATTN_ERR_INVALID_ARG, "B and L must be positive");
    if (B > 65535) return fail(SIGATTN_ERR_UNSUPPORTED, "B must be at most 65535");
    if (!block_size_ok(block_q) || !block_size_ok(block_k))
        return fail(SIGATTN_ERR_UNSUPPORTED, "block sizes must be 32, 64 or 128 (got %d, %d)",
                    block_q, block_k);
    if (mask != nullptr && key_range != nullptr)
        return fail(SIGATTN_ERR_INVALID_ARG, "give an element mask or key ranges, not both");
    if (mask != nullptr && !aligned16(mask))
        return fail(SIGATTN_ERR_ALIGNMENT, "mask is not 16-byte aligned");
    if (key_range != nullptr && (reinterpret_cast<uintptr_t>(key_range) & 7u) != 0)
        return fail(SIGATTN_ERR_ALIGNMENT, "key_range is not 8-byte aligned");
    if (schedule != nullptr) {
        const int64_t need = sigattn_schedule_bytes(B, H, L, block_q, block_k, mask != nullptr);
        if (need < 0) return (int)need;  // its message is set
        if (!aligned16(schedule))
            return fail(SIGATTN_ERR_ALIGNMENT, "schedule is not 16-byte aligned");
        if (schedule_bytes < need)
            return fail(SIGATTN_ERR_INVALID_ARG, "schedule holds %lld bytes, %lld needed",
                        (long long)schedule_bytes, (long long)need);
    }
    const hipStream_t st = (hipStream_t)stream;
    if (schedule != nullptr && mask == nullptr && key_range == nullptr)  // one launch for both
        return launch_status(sigattn::launch_schedule(seq_lens, nullptr, B, H, L, block_q,
                                                      block_k, schedule, st, block_mask),
                             "blockmask_build");
    uint32_t *bits = nullptr;  // with a mask, the schedule also carries it packed to bits
    if (schedule != nullptr && mask != nullptr)
        bits = reinterpret_cast<uint32_t *>(
            static_cast<uint8_t *>(schedule) +
            sigattn::schedule_layout(B, H, L, block_q, block_k, true).bits);
    const int rc = launch_status(sigattn::launch_blockmask(seq_lens, mask, key_range, B, L, block_q,
                                                           block_k, block_mask, st, bits),
                                 "blockmask_build");
    if (rc != SIGATTN_OK || schedule == nullptr) return rc;
    return launch_status(sigattn::launch_schedule(seq_lens, block_mask, B, H, L, block_q, block_k,
                                                  schedule, st),
                         "blockmask_build (schedule)");
}

int sigattn_fwd(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                const int32_t *seq_lens, const uint8_t *block_mask, const void *schedule,
                const uint8_t *mask, const int32_t *key_range, int32_t bias_mode,
                int32_t variant, void *o, float *lse, void *stream) {
    sigattn::AttnParams p = {};
    const void *inputs[3] = {q, k, v};
    void *outputs[1] = {o};
    int st = check_attention(shape, inputs, 3, outputs, 1, seq_lens, block_mask, schedule, mask,
                             key_range, bias_mode, variant, &p);
    if (st != SIGATTN_OK) return st;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return fail(SIGATTN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    return launch_status(sigattn::launch_fwd(p, (hipStream_t)stream), "sigattn_fwd");
}

int sigattn_fwd_noalloc(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                        const int32_t *seq_lens, const uint8_t *block_mask, const uint8_t *mask,
                        const int32_t *key_range, int32_t bias_mode, int32_t variant, void *o,
                        float *lse, void *stream) {
    if (block_mask == nullptr)
        return fail(SIGATTN_ERR_INVALID_ARG, "sigattn_fwd_noalloc needs the block mask");
    sigattn::AttnParams p = {};
    const void *inputs[3] = {q, k, v};
    void *outputs[1] = {o};
    int st = check_attention(shape, inputs, 3, outputs, 1, seq_lens, block_mask, nullptr, mask,
                             key_range, bias_mode, variant, &p);
    if (st != SIGATTN_OK) return st;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return fail(SIGATTN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    const sigattn::ScheduleLayout lay =
        sigattn::schedule_layout(shape->B, shape->H, shape->L, shape->block_q, shape->block_k);
    if (lay.bytes > SIGATTN_NOALLOC_SCRATCH_BYTES)
        return fail(SIGATTN_ERR_UNSUPPORTED,
                    "sigattn_fwd_noalloc: the schedule needs %lld bytes, the library holds %d",
                    (long long)lay.bytes, SIGATTN_NOALLOC_SCRATCH_BYTES);
    hipError_t err;
    uint8_t *sched = static_cast<uint8_t *>(scratch_ptr(&err));
    if (sched == nullptr) return launch_status(err, "sigattn_fwd_noalloc (scratch address)");
    const hipStream_t hs = (hipStream_t)stream;
    st = launch_status(sigattn::launch_schedule(seq_lens, block_mask, shape->B, shape->H,
                                                shape->L, shape->block_q, shape->block_k, sched,
                                                hs),
                       "sigattn_fwd_noalloc (schedule)");
    if (st != SIGATTN_OK) return st;
    p.items1 = reinterpret_cast<const int4 *>(sched + lay.items1);
    p.items2 = reinterpret_cast<const int4 *>(sched + lay.items2);
    p.qlist = reinterpret_cast<const uint32_t *>(sched + lay.qlists);
    p.klist = reinterpret_cast<const uint32_t *>(sched + lay.klists);
    p.qstride = lay.qstride;
    p.kstride = lay.kstride;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    return launch_status(sigattn::launch_fwd(p, hs), "sigattn_fwd_noalloc");
}

int sigattn_diff_fwd(const sigattn_shape *shape, const void *q1, const void *k1, const void *q2,
                     const void *k2, const void *v, const int32_t *seq_lens,
                     const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
                     const int32_t *key_range, int32_t bias_mode, float lambda, void *o, void *o1,
                     void *o2, float *lse1, float *lse2, void *stream) {
    sigattn::AttnParams p = {};
    const void *inputs[5] = {q1, k1, q2, k2, v};
    void *outputs[1] = {o};
    int st = check_attention(shape, inputs, 5, outputs, 1, seq_lens, block_mask, schedule, mask,
                             key_range, bias_mode, SIGATTN_SOFTMAX, &p);
    if (st != SIGATTN_OK) return st;
    if (!isfinite(lambda)) return fail(SIGATTN_ERR_INVALID_ARG, "lambda must be finite");
    if ((reinterpret_cast<uintptr_t>(lse1) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(lse2) & 3u) != 0)
        return fail(SIGATTN_ERR_ALIGNMENT, "lse1/lse2 is not 4-byte aligned");
    if (!aligned16(o1) || !aligned16(o2))
        return fail(SIGATTN_ERR_ALIGNMENT, "o1/o2 is not 16-byte aligned");
    p.v = v;
    p.lambda = lambda;
    if (shape->d == 128) {
        // Two maps' operands and accumulators do not fit one tile loop at
        // d = 128: two softmax passes on the stream.  The first writes map 1's
        // output into o1 (or, without one, into o itself) and its LSE; the
        // second writes map 2's (o2, lse2) and o = O1 - lambda O2 from the
        // first's stored output.
        sigattn::AttnParams p1 = p;
        p1.q = q1;
        p1.k = k1;
        p1.o = o1 != nullptr ? o1 : o;
        p1.lse = lse1;
        p1.variant = sigattn::kSoftmax;
        const hipError_t e = sigattn::launch_fwd(p1, (hipStream_t)stream);
        if (e != hipSuccess) return launch_status(e, "sigattn_diff_fwd");
        sigattn::AttnParams p2 = p;
        p2.q = q2;
        p2.k = k2;
        p2.o = o;
        p2.o1 = p1.o;
        p2.o2 = o2;
        p2.lse = lse2;
        p2.variant = sigattn::kDiffSecond;
        return launch_status(sigattn::launch_fwd(p2, (hipStream_t)stream), "sigattn_diff_fwd");
    }
    p.q = q1;
    p.k = k1;
    p.q2 = q2;
    p.k2 = k2;
    p.o = o;
    p.lse = lse1;
    p.lse2 = lse2;
    p.o1 = o1;
    p.o2 = o2;
    p.variant = sigattn::kDiff;
    return launch_status(sigattn::launch_fwd(p, (hipStream_t)stream), "sigattn_diff_fwd");
}

}  // extern "C"

namespace {

enum BwdParts { kPartDkdv = 1, kPartDq = 2 };

// Differential attention's second map, for the backward that computes both
// maps in one launch (all pointers checked by the caller).
struct SecondMap {
    const void *q2, *k2, *o2;
    const float *lse2;
    void *dq2, *dk2;
    float lambda;
};

int backward(const sigattn_shape *shape, const void *q, const void *k, const void *v,
             const void *dout, const void *o, const float *lse, const int32_t *seq_lens,
             const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
             const int32_t *key_range, int32_t bias_mode, int32_t variant, void *dq, void *dk,
             void *dv, void *stream, int parts, const char *name, float grad_scale = 1.0f,
             bool accumulate_dv = false, void *dv_lo = nullptr,
             const SecondMap *second = nullptr) {
    sigattn::AttnParams p = {};
    const void *inputs[6] = {q, k, v, dout};
    int n_in = 4;
    void *outputs[5];
    int n_out = 0;
    if (parts & kPartDq) outputs[n_out++] = dq;
    if (parts & kPartDkdv) {
        outputs[n_out++] = dk;
        outputs[n_out++] = dv;
    }
    if (second != nullptr) {
        inputs[n_in++] = second->q2;
        inputs[n_in++] = second->k2;
        outputs[n_out++] = second->dq2;
        outputs[n_out++] = second->dk2;
    }
    int st = check_attention(shape, inputs, n_in, outputs, n_out, seq_lens, block_mask, schedule,
                             mask, key_range, bias_mode, variant, &p);
    if (st != SIGATTN_OK) return st;
    if (variant != SIGATTN_SIGMOID) {
        if (o == nullptr || lse == nullptr)
            return fail(SIGATTN_ERR_INVALID_ARG,
                        "the softmax-variant backward needs the forward's o and lse");
        if (!aligned16(o)) return fail(SIGATTN_ERR_ALIGNMENT, "o is not 16-byte aligned");
        if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
            return fail(SIGATTN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
        p.o = const_cast<void *>(o);
        p.lse = const_cast<float *>(lse);
    }
    p.q = q;
    p.k = k;
    p.v = v;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.grad_scale = grad_scale;
    p.accumulate_dv = accumulate_dv ? 1 : 0;
    p.dv_lo = dv_lo;
    if (second != nullptr) {
        p.q2 = second->q2;
        p.k2 = second->k2;
        p.o2 = const_cast<void *>(second->o2);
        p.lse2 = const_cast<float *>(second->lse2);
        p.dq2 = second->dq2;
        p.dk2 = second->dk2;
        p.lambda = second->lambda;
        p.variant = sigattn::kDiff;
    }
    hipStream_t s = (hipStream_t)stream;
    if (parts == (kPartDkdv | kPartDq)) return launch_status(sigattn::launch_bwd(p, s), name);
    if (parts & kPartDkdv) return launch_status(sigattn::launch_bwd_dkdv(p, s), name);
    return launch_status(sigattn::launch_bwd_dq(p, s), name);
}

}  // namespace

extern "C" {

int sigattn_bwd(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                const void *dout, const void *o, const float *lse, const int32_t *seq_lens,
                const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
                const int32_t *key_range, int32_t bias_mode, int32_t variant, void *dq, void *dk,
                void *dv, void *stream) {
    return backward(shape, q, k, v, dout, o, lse, seq_lens, block_mask, schedule, mask,
                    key_range, bias_mode, variant, dq, dk, dv, stream, kPartDkdv | kPartDq,
                    "sigattn_bwd");
}

int sigattn_bwd_dkdv(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                     const void *dout, const void *o, const float *lse,
                     const int32_t *seq_lens, const uint8_t *block_mask, const void *schedule,
                     const uint8_t *mask, const int32_t *key_range, int32_t bias_mode,
                     int32_t variant, void *dk, void *dv, void *stream) {
    return backward(shape, q, k, v, dout, o, lse, seq_lens, block_mask, schedule, mask,
                    key_range, bias_mode, variant, nullptr, dk, dv, stream, kPartDkdv,
                    "sigattn_bwd_dkdv");
}

int sigattn_bwd_dq(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                   const void *dout, const void *o, const float *lse, const int32_t *seq_lens,
                   const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
                   const int32_t *key_range, int32_t bias_mode, int32_t variant, void *dq,
                   void *stream) {
    return backward(shape, q, k, v, dout, o, lse, seq_lens, block_mask, schedule, mask,
                    key_range, bias_mode, variant, dq, nullptr, nullptr, stream, kPartDq,
                    "sigattn_bwd_dq");
}

const char *sigattn_last_error(void) { return g_last_error; }

int sigattn_diff_bwd(const sigattn_shape *shape, const void *q1, const void *k1, const void *q2,
                     const void *k2, const void *v, const void *dout, const void *o1,
                     const void *o2, const float *lse1, const float *lse2,
                     const int32_t *seq_lens, const uint8_t *block_mask, const void *schedule,
                     const uint8_t *mask, const int32_t *key_range, int32_t bias_mode,
                     float lambda, void *dq1, void *dk1, void *dq2, void *dk2, void *dv,
                     void *stream) {
    // Everything the second pass needs is checked before the first is enqueued.
    if (!isfinite(lambda)) return fail(SIGATTN_ERR_INVALID_ARG, "lambda must be finite");
    const void *second[7] = {q2, k2, o2, lse2, dq2, dk2, dv};
    for (const void *ptr : second)
        if (ptr == nullptr)
            return fail(SIGATTN_ERR_INVALID_ARG, "the second map's tensors must not be NULL");
    if (!aligned16(q2) || !aligned16(k2) || !aligned16(o2) || !aligned16(dq2) || !aligned16(dk2))
        return fail(SIGATTN_ERR_ALIGNMENT, "a second-map tensor is not 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse2) & 3u) != 0)
        return fail(SIGATTN_ERR_ALIGNMENT, "lse2 is not 4-byte aligned");
    if (shape != nullptr && shape->d == 64) {
        // Both maps in one pass: each work item holds both maps' operands,
        // dP = dO V^T serves both, and dV takes the weights P1 - lambda P2.
        const SecondMap second = {q2, k2, o2, lse2, dq2, dk2, lambda};
        return backward(shape, q1, k1, v, dout, o1, lse1, seq_lens, block_mask, schedule, mask,
                        key_range, bias_mode, SIGATTN_SOFTMAX, dq1, dk1, dv, stream,
                        kPartDkdv | kPartDq, "sigattn_diff_bwd", 1.0f, false, nullptr, &second);
    }
    // d = 128: two passes.  Map 1: the softmax backward of (Q1, K1) with dO writes dq1, dk1 and dv,
    // and dv's rounding residual into dk2 (written for real only by map 2).
    int st = backward(shape, q1, k1, v, dout, o1, lse1, seq_lens, block_mask, schedule, mask,
                      key_range, bias_mode, SIGATTN_SOFTMAX, dq1, dk1, dv, stream,
                      kPartDkdv | kPartDq, "sigattn_diff_bwd", 1.0f, false, dk2);
    if (st != SIGATTN_OK) return st;
    // Map 2 enters the output as -lambda O2: its gradients are -lambda times
    // the softmax backward of (Q2, K2) with dO, and its dV adds to map 1's
    // (dv plus the residual, each row read before the row's dk2 is written).
    return backward(shape, q2, k2, v, dout, o2, lse2, seq_lens, block_mask, schedule, mask,
                    key_range, bias_mode, SIGATTN_SOFTMAX, dq2, dk2, dv, stream,
                    kPartDkdv | kPartDq, "sigattn_diff_bwd", -lambda, true, dk2);
}

}  // extern "C"
