/*
 * sigattn.h - C ABI of libsigattn.so: fused, tiled attention over padded
 * variable-length batches on AMD Instinct MI355X (gfx950).
 *
 * Operation (per batch entry b, head h; n = clamp(seq_lens[b], 0, L)):
 *   valid(r, c) = r < n and c < n and (mask == NULL or mask[b, r, c] != 0)
 *                 and (key_range == NULL or lo <= c <= hi, with
 *                      (lo, hi) = key_range[b, r, 0..1])
 *                 and (block_mask == NULL or its entry for the tile of (r, c) is non-zero)
 *   s[r, c]     = scale * <q_r, k_c> + beta
 *   beta        = 0 (NONE), -ln n (LOG_SEQLEN), -ln L (LOG_PADLEN)
 *   SIGMOID     o_r = sum_c sigma(s[r, c]) v_c
 *               ("Better Models, Faster Training: Sigmoid Attention for
 *               single-cell Foundation Models", section 2.A, with the bias
 *               b = -log(n) of the same section)
 *   SOFTMAX     o_r = sum_c exp(s) v_c / sum_c exp(s)     (Flash Attention page,
 *               "the mathematics"; computed with a running max and sum)
 *   SOFTMAX1    o_r = sum_c exp(s) v_c / (1 + sum_c exp(s))  (softmax_1 /
 *               QuietAttention page, "Proposition")
 * Sums run over valid (r, c) only.  Padded query rows (r >= n) and rows with
 * no valid key produce exactly zero output and zero gradients.  The content
 * of padded rows of Q, K, V and dO is never read, so it may hold anything,
 * NaN included.
 *
 * Tiles that the binary block mask marks 0 are skipped without loading
 * anything ("Binary Block Masking", "Presentation" / "How it works"; padded
 * blocks on the query and key sides, single-cell page section 2.C).
 *
 * Conventions shared by every entry point:
 * - Device pointers are marked [device], host pointers [host].  The caller
 *   owns every buffer.  The library allocates nothing and never
 *   synchronises: each call enqueues its kernels on `stream` (a hipStream_t;
 *   NULL is the default stream) and returns.  Inputs are never modified.
 * - Return value: SIGATTN_OK or a negative sigattn_status.  Argument errors
 *   are detected on the host before anything is enqueued; SIGATTN_ERR_LAUNCH
 *   reports a failed kernel launch.  sigattn_last_error() gives a message for
 *   the last failure on the calling thread.
 * - seq_lens lives in device memory, so its values are not checked on the
 *   host; kernels clamp each length into [0, L].
 * - An element mask comes in one of two forms, never both in one call:
 *     mask       [device] uint8 [B, L, L], non-zero = may attend (any pattern);
 *     key_range  [device] int32 [B, L, 2], 8-byte aligned: query row r of
 *                batch entry b attends the keys lo <= c <= hi (inclusive,
 *                empty when lo > hi).  This covers the masks whose rows are
 *                intervals (causal, packed documents, causal packed
 *                documents, sliding windows) in 8 bytes per row; the kernels
 *                evaluate it per tile and never read an L x L mask (Binary
 *                Block Masking, "Applications and real-world tests", counts
 *                packed-sequence masks among its targets).
 *   Either form needs a block mask from blockmask_build with the same form.
 */
#ifndef SIGATTN_H
#define SIGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SIGATTN_SIGMOID = 0,
    SIGATTN_SOFTMAX = 1,
    SIGATTN_SOFTMAX1 = 2
} sigattn_variant;

typedef enum {
    SIGATTN_BIAS_NONE = 0,
    SIGATTN_BIAS_LOG_SEQLEN = 1, /* beta = -ln(n), n the unpadded length of the sequence */
    SIGATTN_BIAS_LOG_PADLEN = 2  /* beta = -ln(L), L the padded length */
} sigattn_bias_mode;

typedef enum {
    SIGATTN_OK = 0,
    SIGATTN_ERR_INVALID_ARG = -1, /* null required pointer, non-positive size, bad enum */
    SIGATTN_ERR_UNSUPPORTED = -2, /* head dim or block size not built, sizes or strides
                                     beyond the limits below */
    SIGATTN_ERR_ALIGNMENT = -3,   /* pointer or stride not 16-byte aligned */
    SIGATTN_ERR_LAUNCH = -4       /* HIP reported an error while enqueuing */
} sigattn_status;

/* Largest padded length accepted together with an element mask: the kernels
 * address a batch entry's L x L mask (plus one tile of rows) with 32-bit
 * offsets. */
#define SIGATTN_MAX_MASKED_L 46080

/* Bound on the workgroups of one launch (2^24: times 256 threads, the
 * 32-bit grid limit). */
#define SIGATTN_MAX_WORKGROUPS 16777216

/* Largest row stride (stride_l, o_stride_l) in elements: the kernels address
 * the rows of one tile from its first row with 32-bit byte offsets. */
#define SIGATTN_MAX_ROW_STRIDE 4194304

/*
 * Problem shape.  Q, K, V and dO share one layout, O, dQ, dK and dV another;
 * both are [B, H, L, d] with the head dimension contiguous (stride 1) and the
 * other strides given in elements.  A zero o_stride_* triple means "same as
 * the input strides".  Every base pointer and every stride must be a multiple
 * of 16 bytes (8 bf16 elements).
 */
/* Sizes: B, H <= 65535; 16 * ceil(B * H / 8) * ceil(L / 128) <
 * SIGATTN_MAX_WORKGROUPS (the workgroups of the largest launch, 256 threads
 * each, within HIP's 32-bit grid); row strides at most
 * SIGATTN_MAX_ROW_STRIDE.  Larger problems are UNSUPPORTED and are split by
 * the caller (along B or H: the work is independent). */
typedef struct {
    int32_t B, H, L, d;       /* batch, heads, padded length, head dim (64 or 128) */
    int64_t stride_b, stride_h, stride_l;       /* Q, K, V, dO */
    int64_t o_stride_b, o_stride_h, o_stride_l; /* O, dQ, dK, dV (0,0,0: as inputs) */
    float scale;              /* score scale; <= 0 selects 1/sqrt(d) */
    int32_t block_q, block_k; /* block-mask tile: 32, 64 or 128 rows / columns */
} sigattn_shape;

/*
 * sigattn_schedule_bytes - size in bytes of the schedule buffer that
 * blockmask_build can fill for a batch of B sequences with H heads, padded
 * length L and the given block sizes (see blockmask_build), or a negative
 * sigattn_status: INVALID_ARG (B, H or L <= 0), UNSUPPORTED (block size,
 * sizes beyond the limits of sigattn_shape).  48 bytes per 128-row tile of
 * every (batch entry, head) (the (batch entry, head) pairs rounded up to a
 * multiple of 8), plus 4 * B * ceil(L / 128) * (Tq + Tk + 2); with
 * dense_mask != 0 (a schedule for a batch with an element mask), rounded up
 * to 16 bytes plus 4 * B * L * ceil(L / 32) for the mask packed to bits.
 */
int64_t sigattn_schedule_bytes(int32_t B, int32_t H, int32_t L, int32_t block_q,
                               int32_t block_k, int32_t dense_mask);

/*
 * blockmask_build - binary block matrix of one batch (Binary Block Masking,
 * "Presentation": keep a block when it holds at least one active element;
 * built once, in parallel, and shared by every head and layer), and
 * optionally the work schedule derived from it.
 *
 *   seq_lens    [device] int32 [B]
 *   mask        [device] uint8 [B, L, L] row-major, non-zero = may attend;
 *               NULL for padding-only batches.  Must be 16-byte aligned.
 *   key_range   [device] int32 [B, L, 2] (see above) or NULL; at most one of
 *               mask and key_range.
 *   H           heads of the attention calls the schedule will serve (read
 *               only when schedule is not NULL)
 *   block_mask  [device] uint8 [B, Tq, Tk] output, Tq = ceil(L / block_q),
 *               Tk = ceil(L / block_k); every entry is written with 0, 1 or 3.
 *   schedule    [device] output of schedule_bytes bytes (at least
 *               sigattn_schedule_bytes(B, H, L, block_q, block_k,
 *               mask != NULL)), 16-byte aligned, or NULL for none.
 * Bit 0 of entry (b, i, j) is the binary block matrix: 1 iff some r in
 * [i*block_q, min((i+1)*block_q, L)) and c in [j*block_k, min((j+1)*block_k, L))
 * is valid (definition above without the block-mask term).  Bit 1 marks a full
 * tile (the same page: runs of non-zero blocks need fewer checks): the whole
 * block_q x block_k tile lies inside [0, n) x [0, n) and every element of it
 * is valid; the attention kernels then read no element mask for it.  With
 * mask == NULL bit 0 is i*block_q < n && j*block_k < n and bit 1 is
 * (i+1)*block_q <= n && (j+1)*block_k <= n.
 * With key_range the builder reads only the ranges (O(block_q) work per
 * entry, no L x L scan).
 *
 * The schedule ("How it works": only the runs of kept blocks are visited)
 * holds, for the attention calls of this batch:
 *   - work items: which (batch entry, head, 128-row tile) each workgroup of a
 *     forward or backward launch takes.  Workgroup i runs on XCD i % 8; XCD x
 *     takes the (length rank, head) pairs x, x + 8, ... from the longest
 *     sequence down (ties by batch index; batches of more than 1024 entries
 *     in index order), then the tiles of empty sequences.  Each item carries
 *     its clamped length n.
 *   - kept-entry lists: per batch entry and 128-row group of queries, the
 *     block-mask entries that some block row of the group keeps, in
 *     increasing order, with the rows that keep them and mark them full; per
 *     128-key group the same down the block columns.
 *   - with a mask: the mask packed to one bit per entry (the scan that
 *     builds the block mask reads every valid byte anyway), which the
 *     attention kernels then read instead of the mask's bytes: 4 bytes per
 *     32 entries, one conversion for all heads and layers.
 * Passing it to the attention calls (with this block_mask, and the same mask)
 * spares every workgroup the ranking of the lengths and the scan of
 * block-mask lines; the results are bit for bit those without it.  It stays
 * valid while seq_lens, the mask, H and the block sizes are unchanged, and
 * serves every layer.  A schedule built without a mask must not be passed
 * together with a mask (it holds no packed mask).
 * Errors: INVALID_ARG (null seq_lens/block_mask, B or L <= 0, both mask and
 * key_range, with a schedule: H <= 0 or schedule_bytes too small),
 * UNSUPPORTED (block size not 32/64/128, sizes beyond the limits), ALIGNMENT
 * (mask or schedule not 16-byte, key_range not 8-byte aligned), LAUNCH.
 */
int blockmask_build(const int32_t *seq_lens, const uint8_t *mask, const int32_t *key_range,
                    int32_t B, int32_t H, int32_t L, int32_t block_q, int32_t block_k,
                    uint8_t *block_mask, void *schedule, int64_t schedule_bytes, void *stream);

/*
 * sigattn_fwd - forward pass (single-cell page section 2.C: one fused kernel,
 * block-sparse over padding; Flash Attention page: tiles staged on chip, K/V
 * streamed, online softmax for the softmax variants).
 *
 *   shape       [host]   see sigattn_shape
 *   q, k, v     [device] bf16 [B, H, L, d] (input layout)
 *   seq_lens    [device] int32 [B]
 *   block_mask  [device] uint8 [B, Tq, Tk] from blockmask_build with the same
 *               block sizes, or NULL: tiles are then chosen from seq_lens
 *               alone.  Required with mask or key_range.  Tiles with a zero entry
 *               are skipped; bit 1 set promises a full tile (see
 *               blockmask_build), so a caller's own 0/1 matrix is also valid.
 *   schedule    [device] the schedule blockmask_build wrote together with
 *               block_mask (same seq_lens, mask, H and block sizes), or NULL
 *               (each workgroup then finds its work from seq_lens and
 *               block_mask).  Needs block_mask.
 *   mask        [device] uint8 [B, L, L] or NULL (element mask, all heads;
 *               non-zero = may attend; rows need no alignment); with a mask,
 *               L <= SIGATTN_MAX_MASKED_L (else UNSUPPORTED)
 *   key_range   [device] int32 [B, L, 2] or NULL (key ranges, all heads; see
 *               above); at most one of mask and key_range
 *   o           [device] bf16 [B, H, L, d] (output layout), fully written
 *   lse         [device] float [B, H, L] contiguous, or NULL.  Softmax
 *               variants write the natural log of each row's denominator
 *               (-inf for padded rows and, for SOFTMAX, rows without a valid
 *               key); SIGMOID does not write it.
 * Accumulation is fp32; the weights are rounded to bf16 before the product
 * with V and the output is rounded to bf16 (round to nearest even).
 * Errors: INVALID_ARG (also: both mask and key_range, or either without a
 * block mask), UNSUPPORTED (d not 64/128, block size), ALIGNMENT, LAUNCH.
 */
int sigattn_fwd(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                const int32_t *seq_lens, const uint8_t *block_mask, const void *schedule,
                const uint8_t *mask, const int32_t *key_range, int32_t bias_mode,
                int32_t variant, void *o, float *lse, void *stream);

/*
 * sigattn_bwd - gradients dQ, dK, dV of sum(dO * O)
 * (single-cell page section 2.C: two kernels, one for dQ and one for dK/dV,
 * no atomics, scores and weights recomputed on the fly; section 2.B: the
 * Jacobian of sigmoid attention is diagonal, dS = dP * sigma * (1 - sigma)).
 * For SOFTMAX and SOFTMAX1 the weights are recomputed from the forward's
 * log-sum-exp, P = exp(s - lse), and dS = P * (dP - D) with
 * D = rowsum(dO * O) (the softmax Jacobian; softmax_1 note, "Properties of
 * softmax_1": the derivative of softmax_1 has the same form).
 *
 *   q, k, v, dout   [device] bf16 [B, H, L, d] (input layout)
 *   o               [device] bf16 [B, H, L, d] (output layout): the forward
 *                   output of the same call; required for SOFTMAX and
 *                   SOFTMAX1, ignored (may be NULL) for SIGMOID
 *   lse             [device] fp32 [B, H, L] contiguous: the forward's
 *                   log-sum-exp; same rule as o
 *   seq_lens, block_mask, schedule, mask, key_range: as for sigattn_fwd
 *   dq, dk, dv      [device] bf16 [B, H, L, d] (output layout), fully written;
 *                   rows >= n are 0.
 * bias_mode and variant must be those the forward ran with.
 * The dK/dV and dQ work items write disjoint outputs and use no atomics, so
 * results are bit-for-bit reproducible and equal to those of the two calls
 * below.  When block_q == block_k, both kinds of work item go out in one
 * launch, sharing one ramp-up and one tail; otherwise this is the two
 * launches below.
 * Errors: as sigattn_fwd; INVALID_ARG for a softmax variant without o or
 * lse, ALIGNMENT for o not 16-byte or lse not 4-byte aligned.
 */
int sigattn_bwd(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                const void *dout, const void *o, const float *lse, const int32_t *seq_lens,
                const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
                const int32_t *key_range, int32_t bias_mode, int32_t variant, void *dq,
                void *dk, void *dv, void *stream);

/*
 * sigattn_bwd_dkdv / sigattn_bwd_dq - the two halves of sigattn_bwd, each one
 * kernel launch (single-cell page section 2.C: the backward pass is split
 * into a kernel for the K/V gradients and a kernel for the Q gradients).
 * Arguments, layouts and errors as sigattn_bwd; sigattn_bwd_dkdv writes only
 * dk and dv, sigattn_bwd_dq writes only dq.  Useful when only one side needs
 * gradients, and to time the two kernels apart.
 */
int sigattn_bwd_dkdv(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                     const void *dout, const void *o, const float *lse,
                     const int32_t *seq_lens, const uint8_t *block_mask, const void *schedule,
                     const uint8_t *mask, const int32_t *key_range, int32_t bias_mode,
                     int32_t variant, void *dk, void *dv, void *stream);
int sigattn_bwd_dq(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                   const void *dout, const void *o, const float *lse, const int32_t *seq_lens,
                   const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
                   const int32_t *key_range, int32_t bias_mode, int32_t variant, void *dq,
                   void *stream);

/*
 * sigattn_fwd_noalloc - sigattn_fwd with its work schedule kept in memory the
 * library holds, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * It builds the schedule (see blockmask_build) from seq_lens and block_mask
 * into a static device array of SIGATTN_NOALLOC_SCRATCH_BYTES bytes (one per
 * GPU, held until the process ends; its address is looked up once per device
 * on the first call there), then runs the forward with it.  It calls no
 * allocator.  Results equal sigattn_fwd's with a schedule from
 * blockmask_build, bit for bit.
 * Arguments as sigattn_fwd (no schedule argument); block_mask is required.
 * Every call on one GPU uses that GPU's one array, whatever the stream:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race and must be ordered by the caller; calls in one stream are ordered.
 * Errors: as sigattn_fwd; INVALID_ARG for a NULL block_mask; UNSUPPORTED when
 * the schedule (sigattn_schedule_bytes(B, H, L, block_q, block_k, 0)) exceeds
 * SIGATTN_NOALLOC_SCRATCH_BYTES; LAUNCH also when the array's address cannot
 * be obtained.
 */
#define SIGATTN_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
int sigattn_fwd_noalloc(const sigattn_shape *shape, const void *q, const void *k, const void *v,
                        const int32_t *seq_lens, const uint8_t *block_mask, const uint8_t *mask,
                        const int32_t *key_range, int32_t bias_mode, int32_t variant, void *o,
                        float *lse, void *stream);

/*
 * sigattn_diff_fwd - differential attention forward ("Differential
 * Transformer" note, "How differential attention works"): two softmax maps
 * over one value tensor, the second subtracted with the scalar lambda,
 *   o_r = sum_c softmax_c(s1[r, c]) v_c - lambda * sum_c softmax_c(s2[r, c]) v_c,
 *   s_i[r, c] = scale * <q_i r, k_i c> + beta,
 * over the valid (r, c) of the definition above (the same masks for both
 * maps).  At d = 64 both maps run through one tile loop: each V tile is
 * loaded once and feeds both.  At d = 128 (where two maps' operands do not
 * fit one loop) two softmax passes run on `stream`: the first writes map 1's
 * output to o1, or without one to o, the second combines it with map 2's as
 * o = bf16(O1) - lambda O2, rounded once more.  lambda is the layer's scalar as a plain input (its
 * reparametrisation and the per-head normalisation after the attention
 * belong to the model, not here).
 *
 *   q1, k1, q2, k2, v  [device] bf16 [B, H, L, d] (input layout), as q, k, v
 *                      of sigattn_fwd
 *   seq_lens, block_mask, schedule, mask, key_range, bias_mode: as for sigattn_fwd
 *                      (the bias cancels in each softmax; it shifts the LSEs)
 *   lambda             [host] finite float
 *   o                  [device] bf16 [B, H, L, d] (output layout), fully
 *                      written; padded rows and rows without a valid key are 0
 *   o1, o2             [device] bf16 [B, H, L, d] (output layout) or NULL: each
 *                      map's own output softmax(S_i) V, fully written when
 *                      given (sigattn_diff_bwd needs them)
 *   lse1, lse2         [device] fp32 [B, H, L] contiguous, or NULL: each map's
 *                      log-sum-exp, as sigattn_fwd's SOFTMAX lse
 * Errors: as sigattn_fwd; INVALID_ARG for a non-finite lambda, ALIGNMENT for
 * o1 or o2 not 16-byte, lse1 or lse2 not 4-byte aligned.
 */
int sigattn_diff_fwd(const sigattn_shape *shape, const void *q1, const void *k1, const void *q2,
                     const void *k2, const void *v, const int32_t *seq_lens,
                     const uint8_t *block_mask, const void *schedule, const uint8_t *mask,
                     const int32_t *key_range, int32_t bias_mode, float lambda, void *o, void *o1,
                     void *o2, float *lse1, float *lse2, void *stream);

/*
 * sigattn_diff_bwd - gradients of sum(dO * O) for O = O1 - lambda O2 of
 * sigattn_diff_fwd.  The output is linear in the two maps, so each map's
 * gradients are those of a softmax attention with dO (map 1) or -lambda dO
 * (map 2), and dV is the sum of both (sigattn_bwd's softmax backward: P from
 * the map's LSE, dS = P * (dP - D), D = rowsum(dO * O_i) with the map's own
 * output O_i).  No atomics are used and results are reproducible.  At
 * d = 64 both maps run in one launch: each work item computes both maps'
 * scores, dP = dO V^T once for both, and dV from the weights P1 - lambda P2
 * (rounded to bf16 once).  At d = 128 two launches on `stream`; the second
 * adds its dV to the first's.  Between the two, map 1's dV is held as bf16
 * plus its bf16 rounding residual (kept in dk2's storage, which the second
 * launch then overwrites with dK2), so the sum is formed in fp32 from ~16
 * significant bits of each term.
 *
 *   q1, k1, q2, k2, v, dout  [device] bf16 [B, H, L, d] (input layout)
 *   o1, o2, lse1, lse2       the forward's per-map outputs and LSEs (required)
 *   seq_lens, block_mask, schedule, mask, key_range, bias_mode, lambda: as for
 *                            the forward
 *   dq1, dk1, dq2, dk2, dv   [device] bf16 [B, H, L, d] (output layout), fully
 *                            written; rows >= n are 0
 * Errors: as sigattn_bwd; INVALID_ARG for a NULL tensor or a non-finite
 * lambda (all checked before anything is enqueued).
 */
int sigattn_diff_bwd(const sigattn_shape *shape, const void *q1, const void *k1, const void *q2,
                     const void *k2, const void *v, const void *dout, const void *o1,
                     const void *o2, const float *lse1, const float *lse2,
                     const int32_t *seq_lens, const uint8_t *block_mask, const void *schedule,
                     const uint8_t *mask, const int32_t *key_range, int32_t bias_mode,
                     float lambda, void *dq1, void *dk1, void *dq2, void *dk2, void *dv,
                     void *stream);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char *sigattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SIGATTN_H */
