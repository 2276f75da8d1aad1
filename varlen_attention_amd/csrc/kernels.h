// Parameter blocks and launchers of the gfx950 kernels.  The host ABI layer
// (api.hip) validates arguments and calls these; each launcher enqueues its
// kernels on the given stream and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sigattn {

// The ABI's variants, plus kDiff: differential attention, two softmax maps
// over one V combined as O1 - lambda O2 (set by the differential entry
// points), and kDiffSecond: its forward's second pass where the two maps do
// not fit one tile loop (d = 128), a softmax map whose store combines its
// output with the first map's stored output.
enum Variant { kSigmoid = 0, kSoftmax = 1, kSoftmax1 = 2, kDiff = 3, kDiffSecond = 4 };

// Layout of a schedule buffer (blockmask_build's optional output; byte
// offsets from its start).  Work items are 16 bytes: {b, h, tile | kind << 30,
// n}, tile = -1 past the last item.  A launch over one kind of 128-row tile
// (forward, dK/dV alone, dQ alone) reads items1, the one-launch backward
// items2; slot i is workgroup i's item, and workgroup i runs on XCD i % 8.
// An item whose tile starts at or past n is a zero item: it writes the zero
// rows of tiles tile .. tile + kZeroTiles - 1 (below L) and nothing else;
// an XCD's zero items follow its compute items (items1, when they are not
// more numerous; else spread between them) or are spread over the second
// half of them (items2).
// Entry lists hold, per batch entry and 128-row group of queries (qlists) or
// keys (klists), a count word and then one word per block-mask entry that
// some line of the group keeps: e | kept-by-line << 24 | full-by-line << 28,
// in increasing e (lines: the block rows, or columns, the group spans).
// A schedule built with a dense element mask ends with that mask packed to
// bits: per batch entry and query row, words_per_row words, bit t of word w
// the entry for key 32 w + t (rows and keys below n; the rest unspecified).
// Fully padded 128-row tiles per zero item of a schedule.
constexpr int kZeroTiles = 4;

struct ScheduleLayout {
    int64_t slots1, slots2;  // items in the two arrays
    int64_t items1, items2;  // byte offsets of the item arrays
    int64_t qlists, klists;  // byte offsets of the entry lists
    int64_t bits;            // byte offset of the packed mask (dense_mask layouts)
    int64_t bytes;           // the whole buffer
    int groups;              // 128-row groups along L
    int qstride, kstride;    // words per query group (1 + Tk) and key group (1 + Tq)
    int words_per_row;       // packed mask: ceil(L / 32)
};

__host__ __device__ inline ScheduleLayout schedule_layout(int B, int H, int L, int block_q,
                                                          int block_k, bool dense_mask = false) {
    ScheduleLayout s;
    const int64_t G = ((int64_t)L + 127) / 128;
    const int64_t Tq = ((int64_t)L + block_q - 1) / block_q;
    const int64_t Tk = ((int64_t)L + block_k - 1) / block_k;
    s.groups = (int)G;
    s.qstride = (int)(1 + Tk);
    s.kstride = (int)(1 + Tq);
    s.slots1 = 8 * (((int64_t)B * H + 7) / 8) * G;
    s.slots2 = 2 * s.slots1;
    s.items1 = 0;
    s.items2 = 16 * s.slots1;
    s.qlists = s.items2 + 16 * s.slots2;
    s.klists = s.qlists + 4 * (int64_t)B * G * s.qstride;
    s.bits = (s.klists + 4 * (int64_t)B * G * s.kstride + 15) / 16 * 16;
    s.words_per_row = (int)(((int64_t)L + 31) / 32);
    s.bytes = dense_mask ? s.bits + 4 * (int64_t)B * L * s.words_per_row
                         : s.klists + 4 * (int64_t)B * G * s.kstride;
    return s;
}

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
    // Backward: bf16 [B, H, L, d] (output layout) holding the rounding residual
    // of dv, or null.  Without accumulate_dv the store writes dv = bf16(x) and
    // dv_lo = bf16(x - dv); with it, the value added to is dv + dv_lo, so a
    // sum over two launches keeps ~16 significant bits between them.
    void *dv_lo;
    const int32_t *seq_lens;        // [B]
    const uint8_t *block_mask;      // [B, Tq, Tk] or null
    const uint8_t *mask;            // [B, L, L] or null
    const int32_t *key_range;       // [B, L, 2] or null (at most one of mask, key_range)
    // With a mask and a schedule: the mask packed to bits in the schedule
    // (ScheduleLayout), bits_w words per row; kernels built for a schedule
    // read these instead of the mask's bytes.
    const uint32_t *mask_bits;
    int bits_w;
    // From a schedule buffer (all null without one): the work items of
    // launches over one kind of tile (items1) and of the one-launch backward
    // (items2), one per workgroup, and the kept-entry lists of query and key
    // groups.
    const int4 *items1, *items2;
    const uint32_t *qlist, *klist;
    int qstride, kstride;           // words per group list
    int64_t sb, sh, sl;             // input strides (elements)
    int64_t osb, osh, osl;          // output strides (elements)
    int B, H, L, d;
    int block_q, block_k, Tq, Tk;   // block-mask geometry
    float scale;
    int bias_mode, variant;
    // Differential forward in two passes (kDiffSecond): o1 holds the first
    // map's output, read at the store; o2, or null, receives the second's.
    // Differential backward in one launch: the second map's gradients (bf16
    // [B, H, L, d], output layout).  Its inputs are q2, k2, o2 (the map's own
    // forward output) and lse2; the first map's are q, k, o and lse.
    void *dq2, *dk2;
};

// bits_out (or null; with mask): the mask packed to bits, ScheduleLayout's
// words_per_row words per row.
hipError_t launch_blockmask(const int32_t *seq_lens, const uint8_t *mask,
                            const int32_t *key_range, int B, int L, int block_q, int block_k,
                            uint8_t *out, hipStream_t stream, uint32_t *bits_out = nullptr);
// Work items and kept-entry lists (ScheduleLayout) from seq_lens and a
// finished block mask, enqueued after it on the same stream; or, with
// padding_mask_out, for a padding-only batch: the block mask written into
// padding_mask_out and the schedule in the same launch (block_mask unused).
hipError_t launch_schedule(const int32_t *seq_lens, const uint8_t *block_mask, int B, int H,
                           int L, int block_q, int block_k, void *schedule, hipStream_t stream,
                           uint8_t *padding_mask_out = nullptr);
hipError_t launch_fwd(const AttnParams &p, hipStream_t stream);
hipError_t launch_bwd_dkdv(const AttnParams &p, hipStream_t stream);
hipError_t launch_bwd_dq(const AttnParams &p, hipStream_t stream);
// dK, dV and dQ in one launch (two launches when the tile heights differ).
hipError_t launch_bwd(const AttnParams &p, hipStream_t stream);

}  // namespace sigattn
