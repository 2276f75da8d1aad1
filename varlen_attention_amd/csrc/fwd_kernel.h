// Forward kernel template (included by one translation unit per variant):
// fused, tiled attention over a padded variable-length batch
// for gfx950 (sigmoid, online softmax and softmax_1 through one tile loop, and
// differential attention: two softmax maps over one V, "Differential
// Transformer" note, "How differential attention works").
//
// Method: "Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", section 2.A (sigma(QK^T/sqrt(d) + b) V, b = -log n) and
// 2.C (one fused kernel, block-sparse skipping of padded blocks on both
// sides); Binary Block Masking ("How it works": only blocks with an active
// entry are processed); Flash Attention page ("the algorithm", "the
// mathematics": K/V tiles staged on chip, running max and sum merged by
// exp(m_old - m_new)).
//
// Work decomposition: a workgroup of NW waves owns BQ = 32*NW query rows of one
// (batch entry, head); each wave owns 32 rows.  Key tiles of BK = 32*KB rows
// are visited in increasing order; a tile whose block-mask entry is 0 is never
// loaded.  Per tile:
//   S^T = K Q^T           32x32x16 bf16 MFMA; K rows from LDS, Q in registers
//   P^T = f(S^T)          epilogue in registers (sigmoid, or online softmax)
//   O^T += V^T P^T        P^T stays in registers as the B operand; V^T is read
//                         from the row-major V tile with transposing LDS reads
// Computing the transposed products puts one query per lane (lane % 32), so
// softmax row statistics are lane-local plus one exchange with lane ^ 32.
// K and V tiles are double-buffered in LDS: the next tile's rows are fetched
// into registers while the current tile computes, then written to the other
// buffer, with one barrier per tile.  An element mask (dense bytes or key
// ranges) is staged per tile as bits in LDS next to K and V (MaskStage /
// RangeStage); full tiles (block-mask bit 1) need none, and a wave whose
// share of a tile keeps nothing skips it.  Fully padded query tiles only
// write zeros.
#pragma once

#include <initializer_list>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace sigattn {

namespace {

// LDS row strides (elements).  K rows are read 16 bytes per lane down 32 rows:
// a stride of 4 banks (mod 32) spreads 8 rows over all banks.  V rows are read
// 8 bytes per lane, 4 rows x 32 bytes per 16 lanes: a stride of 8 banks.
template <int D> struct Pad { static constexpr int K = D + 8, V = D + 16; };

template <int D, int BK, int NT, int NK = 1>
struct KVStage {
    // Each thread moves CH 16-byte chunks of each of the NK key tiles and of
    // V per tile.  Offsets are loop-invariant; the per-tile part lives in the
    // buffer descriptors.
    static constexpr int kChunksPerRow = D / 8;
    static constexpr int CH = BK * kChunksPerRow / NT;
    static_assert(CH * NT == BK * kChunksPerRow, "tile must split evenly over threads");
    uint4 k[NK][CH], v[CH];
    int goff[CH], koff[CH], voff[CH];

    __device__ __forceinline__ void init(int64_t sl, int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            const int row = idx / kChunksPerRow, col = (idx % kChunksPerRow) * 8;
            goff[c] = (int)(((int64_t)row * sl + col) * 2);
            koff[c] = row * Pad<D>::K + col;
            voff[c] = row * Pad<D>::V + col;
        }
    }

    // rk[i]: the i-th key tensor's rows; Ks + i * KTILE receives it.
    __device__ __forceinline__ void load(const rsrc_t (&rk)[NK], rsrc_t rv) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
#pragma unroll
            for (int i = 0; i < NK; ++i) k[i][c] = buffer_load16(rk[i], goff[c]);
            v[c] = buffer_load16(rv, goff[c]);
        }
    }

    static constexpr int KTILE = BK * Pad<D>::K;

    __device__ __forceinline__ void store(bf16 *Ks, bf16 *Vs) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
#pragma unroll
            for (int i = 0; i < NK; ++i)
                *reinterpret_cast<uint4 *>(Ks + i * KTILE + koff[c]) = k[i][c];
            *reinterpret_cast<uint4 *>(Vs + voff[c]) = v[c];
        }
    }
};

}  // namespace

// Online softmax: how far (log2 units) a row maximum may pass the reference
// maximum before the running state is rescaled.
constexpr float kLazyRescale = 8.0f;

// Waves per SIMD the register allocation must allow.  One unmasked map at
// d = 64 is held to 128 registers, four waves: the softmax variants would
// otherwise take about 138 and run three (3 % slower).  One map at d = 128
// with 32-key steps is held to 168, three waves: the softmax variants would
// otherwise take up to 204 and run two (15 % slower with key ranges).  Two
// maps (differential attention, d = 64 only) run two waves.
template <int D, int VARIANT, int MASK, int KB>
constexpr int kFwdWavesPerSimd =
    D == 64 && VARIANT != kDiff && MASK == kMaskNone ? 4 : (D == 128 && KB == 1 ? 3 : 2);

// R: block-mask rows per workgroup (BQ / block_q); wave w follows row
// w * R / NW, so smaller block rows keep four waves per workgroup.
// LIST: built for a schedule (work items and kept-entry lists from it).
template <int D, int VARIANT, int NW, int KB, int MASK, int R, bool LIST>
__global__ void __launch_bounds__(64 * NW, (kFwdWavesPerSimd<D, VARIANT, MASK, KB>))
fwd_kernel(const AttnParams p) {
    constexpr bool MASKED = MASK != kMaskNone;
    // Differential attention runs two softmax maps (their own Q, K, running
    // max and sum, and output accumulator) over the same V tiles and mask.
    constexpr int MAPS = VARIANT == kDiff ? 2 : 1;
    constexpr bool kSoft = VARIANT != kSigmoid;
    constexpr int BQ = 32 * NW, BK = 32 * KB, NT = 64 * NW;
    constexpr int KS = D / 16;  // MFMA k-steps over the head dimension
    constexpr int DB = D / 32;  // 32-wide blocks of the head dimension
    constexpr int KP = Pad<D>::K, VP = Pad<D>::V;
    __shared__ __attribute__((aligned(16))) bf16 Ks[2][MAPS * BK * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vs[2][BK * VP];
    __shared__ uint32_t Ms[2][MASKED ? BQ * BK / 32 : 1];  // element-mask bits per tile

    static_assert(BQ == 128, "work items are 128-row tiles");
    int b, h, kind, qt, n;
    if (!work_item<1, LIST>(p, b, h, kind, qt, n)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int L = p.L;
    const int q0 = qt * BQ;
    bf16 *ob = reinterpret_cast<bf16 *>(p.o) + b * p.osb + h * p.osh;
    float *lseb[MAPS];
    lseb[0] = p.lse ? p.lse + ((int64_t)b * p.H + h) * L : nullptr;
    if constexpr (MAPS == 2) lseb[1] = p.lse2 ? p.lse2 + ((int64_t)b * p.H + h) * L : nullptr;

    // Rows [r0, r0 + rows) of a fully padded query tile: zeros (LSE -inf).
    auto zero_tile = [&](int r0, int rows) {
        for (int idx = tid; idx < rows * (D / 8); idx += NT) {
            const int r = r0 + idx / (D / 8), c = (idx % (D / 8)) * 8;
            *reinterpret_cast<uint4 *>(ob + (int64_t)r * p.osl + c) = make_uint4(0, 0, 0, 0);
            if constexpr (MAPS == 2)
                for (void *om : {p.o1, p.o2})
                    if (om != nullptr)
                        *reinterpret_cast<uint4 *>(reinterpret_cast<bf16 *>(om) + b * p.osb +
                                                   h * p.osh + (int64_t)r * p.osl + c) =
                            make_uint4(0, 0, 0, 0);
            if constexpr (VARIANT == kDiffSecond)
                if (p.o2 != nullptr)
                    *reinterpret_cast<uint4 *>(reinterpret_cast<bf16 *>(p.o2) + b * p.osb +
                                               h * p.osh + (int64_t)r * p.osl + c) =
                        make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int mp = 0; mp < MAPS; ++mp)
            if (kSoft && lseb[mp])
                for (int r = r0 + tid; r < r0 + rows; r += NT) lseb[mp][r] = -INFINITY;
    };
    if (q0 >= n) {  // a zero item: zeros, nothing else
        zero_tile(q0, zero_item_rows<BQ, LIST>(q0, L));
        return;
    }

    const bf16 *qb[MAPS], *kb[MAPS];
    qb[0] = reinterpret_cast<const bf16 *>(p.q) + b * p.sb + h * p.sh;
    kb[0] = reinterpret_cast<const bf16 *>(p.k) + b * p.sb + h * p.sh;
    if constexpr (MAPS == 2) {
        qb[1] = reinterpret_cast<const bf16 *>(p.q2) + b * p.sb + h * p.sh;
        kb[1] = reinterpret_cast<const bf16 *>(p.k2) + b * p.sb + h * p.sh;
    }
    const bf16 *vb = reinterpret_cast<const bf16 *>(p.v) + b * p.sb + h * p.sh;
    const int line0 = q0 / p.block_q;  // first block-mask row of this tile
    const uint8_t *bm_row =
        p.block_mask ? p.block_mask + ((int64_t)b * p.Tq + line0) * p.Tk : nullptr;
    // Block rows that exist (with a block mask) or start below n (without).
    const int lines = p.block_mask ? min(R, p.Tq - line0)
                                   : min(R, (n - q0 + p.block_q - 1) / p.block_q);

    const int ql = lane & 31, hh = lane >> 5;
    const int wl = w * R / NW;        // this wave's block-mask row (0 .. R - 1)
    const int qr = q0 + w * 32 + ql;  // this lane's query row
    const bool q_valid = qr < n;
    const MaskSource msrc = mask_source<MASK>(p, b);
    // Per-lane offsets of the transposing V reads (see lds_read_tr4).
    const int trow = 4 * hh + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // Q^T operand: lane holds Q[qr][16 ks + 8 hh .. + 7].
    // Rows >= n read as zeros through the descriptor.
    bf16x8 qreg[MAPS][KS];
#pragma unroll
    for (int mp = 0; mp < MAPS; ++mp) {
        const rsrc_t rq = make_rsrc(qb[mp] + (int64_t)q0 * p.sl, (int64_t)(n - q0) * p.sl * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg[mp][ks] = as_bf16x8(
                buffer_load16(rq, (int)(((int64_t)(w * 32 + ql) * p.sl + ks * 16 + hh * 8) * 2)));
    }

    // SIGMOID: Q is scaled by c1 before the loop, so the S^T accumulator is
    // u = -scale * s * log2 e and the weight is 1 / (1 + exp(-b) 2^u); the
    // weight is rounded to bf16 for the PV product anyway.  Softmax keeps Q
    // as it is and forms t = scale * s * log2 e + b * log2 e in fp32, since
    // the log-sum-exp it returns would inherit the rounding of a scaled Q.
    const float c1 = VARIANT == kSigmoid ? -p.scale * kLog2e : p.scale * kLog2e;
    const float c0 = bias_value(p.bias_mode, n, L) * kLog2e;
    const float cexp = bias_factor(p.bias_mode, n, L);

    f32x16 oacc[MAPS][DB];
    float m_run[MAPS], l_run[MAPS];
#pragma unroll
    for (int mp = 0; mp < MAPS; ++mp) {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[mp][db] = f32x16{};
        m_run[mp] = VARIANT == kSoftmax1 ? 0.0f : -INFINITY;  // log2 domain
        l_run[mp] = (VARIANT == kSoftmax1 && hh == 0) ? 1.0f : 0.0f;  // split over lane halves
    }

    // Descriptors of the K and V rows [k0, n): rows past n read as zeros.
    auto rows_rsrc = [&](const bf16 *base, int k0) {
        return make_rsrc(base + (int64_t)k0 * p.sl, (int64_t)(n - k0) * p.sl * 2);
    };
    // The first active key tile is tile 0 unless the block mask says
    // otherwise, so tile 0 is fetched before the block mask is read and the
    // two memory round trips overlap; another first tile is fetched again.
    // The first stage is written unconditionally (tile 0 when nothing is
    // active, harmless): every path into the loop has then waited for all
    // earlier loads, Q included.
    KVStage<D, BK, NT, MAPS> stage;
    auto load_tile = [&](int t) {
        rsrc_t rk[MAPS];
#pragma unroll
        for (int mp = 0; mp < MAPS; ++mp) rk[mp] = rows_rsrc(kb[mp], t * BK);
        stage.load(rk, rows_rsrc(vb, t * BK));
    };
    stage.init(p.sl, tid);
    load_tile(0);
    MaskStager<MASK, BQ, BK, NT, true> mstage;
    int mcls = kMixed;  // this wave's share of the current tile (element mask)
    if constexpr (MASKED) mstage.init(tid);
    Schedule<BK, R, true, LIST> sched;
    if constexpr (LIST)
        sched.init(p.qlist + ((int64_t)b * ((L + 127) / 128) + qt) * p.qstride, p.Tk, wl, n,
                   p.block_k);
    else
        sched.init(bm_row, p.Tk, lines, wl, n, p.block_k);
    int kt = sched.next();
    const int kt_want = sched.want();
    bool on = kt_want != kWantNone;  // this wave's row keeps the current tile
    if (kt > 0) load_tile(kt);
    if constexpr (MASKED)
        if (kt >= 0) mstage.load(msrc, n, q0, kt * BK, kt_want);
    int buf = 0;
    stage.store(Ks[0], Vs[0]);
    if constexpr (MASKED)
        if (kt >= 0) mcls = mstage.store(Ms[0], q0, kt * BK, n, kt_want);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        if constexpr (VARIANT == kSigmoid) qreg[0][ks] = scale8(qreg[0][ks], c1);
    __syncthreads();

    while (kt >= 0) {
        const int k0 = kt * BK;
        const int nxt = sched.next();
        const int nxt_want = sched.want();
        if (nxt >= 0) load_tile(nxt);
        if constexpr (MASKED)
            if (nxt >= 0) mstage.load(msrc, n, q0, nxt * BK, nxt_want);
        const bf16 *Kc = Ks[buf];
        const bf16 *Vc = Vs[buf];

        // One tile body per kernel instantiation (no second copy for special
        // tiles), so the scheduler can overlap the MFMAs of one key block with
        // the epilogue of another, and the accumulators stay in place across
        // iterations; its only branches are uniform ones around work that
        // most tiles skip.  MODE 0: no per-element masking.  Padded key rows of K and V read as
        // zeros, so for sigmoid their weights multiply zero rows, and padded
        // query rows are zeroed at the store: every padding-only sigmoid tile
        // is MODE 0.  MODE 1: softmax without an element mask (padded keys
        // must not enter the row max and sum).  MODE 2: element mask.
        auto tile = [&](auto mode_tag) {
            constexpr int MODE = decltype(mode_tag)::value;
            // S^T for each map and 32-key block: sacc[mp][kb2][4i + j] is
            // S^T[key k0 + 32 kb2 + 8 i + 4 hh + j][qr].
            f32x16 sacc[MAPS][KB];
#pragma unroll
            for (int mp = 0; mp < MAPS; ++mp)
#pragma unroll
                for (int kb2 = 0; kb2 < KB; ++kb2) {
                    sacc[mp][kb2] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                            Kc + mp * BK * KP + (kb2 * 32 + ql) * KP + ks * 16 + hh * 8);
                        sacc[mp][kb2] = mfma32(a, qreg[mp][ks], sacc[mp][kb2]);
                    }
                }
            // Per-element validity.  MODE 1: key 8 i + 4 hh + j of a 32-key
            // block is valid when 8 i + j < lim: bit 8 i + j of a word with
            // the lim lowest bits set, taken out like a mask bit (bit ops
            // instead of compares, whose condition registers cost wait
            // states).  Padded query rows need no check: their output is
            // zeroed at the store and their LSE set apart.
            uint32_t vw[KB];
            if constexpr (MODE == 1) {
#pragma unroll
                for (int kb2 = 0; kb2 < KB; ++kb2) {
                    const int lim = n - (k0 + kb2 * 32 + hh * 4);
                    vw[kb2] = lim >= 32 ? ~0u : lim <= 0 ? 0u : (1u << lim) - 1u;
                }
            }
            // MODE 2: the tile's mask bits (validity folded in); key
            // 8 i + 4 hh + j of a 32-key block is bit key_bit(8 i + 4 hh + j):
            // 8 j + 2 i + hh (dense) or 8 i + 4 hh + j (ranges).  A wave whose
            // share of the tile keeps every entry (kDense, found when it
            // staged the words) needs no selects; the others turn masked
            // scores into values of weight 0 before the weights (a uniform
            // branch, so the kept tiles pay nothing).
            if constexpr (MODE == 2) {
                if (mcls != kDense) {
                    constexpr bool kDenseBits = MASK == kMaskDense;
#pragma unroll
                    for (int kb2 = 0; kb2 < KB; ++kb2) {
                        const uint32_t mw = Ms[buf][kb2 * BQ + w * 32 + ql] >> (kDenseBits ? hh : 4 * hh);
#pragma unroll
                        for (int mp = 0; mp < MAPS; ++mp)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                sacc[mp][kb2][r] = keep_score<kSoft>(
                                    sacc[mp][kb2][r],
                                    mask_select(mw, kDenseBits ? 8 * (r & 3) + 2 * (r >> 2)
                                                               : 8 * (r >> 2) + (r & 3)));
                    }
                }
            }

            // moff: per map, c0 - m, so that a weight is exp2(s c1 + moff).
            float moff[MAPS];
            if constexpr (kSoft) {
                // Online softmax, per map: tile maximum of the raw scores over
                // this lane's keys and its partner lane's (lane ^ 32).  c1 > 0,
                // and s c1 + c0 rounds monotonically in s, so the maximum of
                // the logits t = s c1 + c0 is the logit of the maximum score.
                // Then rescale the state.
                // MODE 1 masks only the tile that holds key n - 1 (a uniform
                // branch; the tiles before it have no padded key).
                if constexpr (MODE == 1) {
                    if (k0 + BK > n) {
#pragma unroll
                        for (int mp = 0; mp < MAPS; ++mp)
#pragma unroll
                            for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
                                for (int r = 0; r < 16; ++r)
                                    sacc[mp][kb2][r] = keep_bits_or_neg_inf(
                                        sacc[mp][kb2][r], mask_select(vw[kb2], (r >> 2) * 8 + (r & 3)));
                    }
                }
#pragma unroll
                for (int mp = 0; mp < MAPS; ++mp) {
                    float smax = -INFINITY;
#pragma unroll
                    for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            smax = fmaxf(smax, sacc[mp][kb2][r]);
                        }
                    smax = fmaxf(smax, __shfl_xor(smax, 32));
                    const float tmax = fmaf(smax, c1, c0);
                    // The reference m_run moves only when some row's maximum
                    // passes it by more than kLazyRescale (weights stay below
                    // 2^kLazyRescale, harmless in fp32 and bf16): most tiles
                    // then skip rescaling the state.  The sums stay exact
                    // relative to m_run, and so does the log-sum-exp (each
                    // map of differential attention decides for itself).
                    if (__ballot(tmax > m_run[mp] + kLazyRescale) != 0) {
                        const float m_new = fmaxf(m_run[mp], tmax);
                        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
                        const float alpha = __builtin_amdgcn_exp2f(m_run[mp] - m_use);
                        m_run[mp] = m_new;
                        l_run[mp] *= alpha;
#pragma unroll
                        for (int db = 0; db < DB; ++db) oacc[mp][db] *= alpha;
                    }
                    moff[mp] = c0 - (m_run[mp] == -INFINITY ? 0.0f : m_run[mp]);
                }
            }

            // Per 32-key block: weights, then O^T += V^T P^T (two 16-key
            // steps); each V fragment serves every map.
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2) {
                float pv[MAPS][16];
#pragma unroll
                for (int mp = 0; mp < MAPS; ++mp)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        if constexpr (VARIANT == kSigmoid) {
                            pv[mp][r] = sigmoid_scaled(sacc[mp][kb2][r], cexp);
                        } else {
                            pv[mp][r] = __builtin_amdgcn_exp2f(fmaf(sacc[mp][kb2][r], c1, moff[mp]));
                            l_run[mp] += pv[mp][r];
                        }
                    }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 pb[MAPS];
#pragma unroll
                    for (int mp = 0; mp < MAPS; ++mp) pb[mp] = pack8(&pv[mp][kk * 8]);
                    const bf16 *vrow = Vc + (kb2 * 32 + kk * 16 + trow) * VP + tcol;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 a = cat8(lds_read_tr4(vrow + db * 32),
                                              lds_read_tr4(vrow + 8 * VP + db * 32));
#pragma unroll
                        for (int mp = 0; mp < MAPS; ++mp)
                            oacc[mp][db] = mfma32(a, pb[mp], oacc[mp][db]);
                    }
                }
            }
        };
        if constexpr (MASKED) {
            // The wave's rows of this tile, as found when it staged them:
            // nothing kept means no work.  (A second, unmasked copy of the
            // body for tiles whose entries are all kept measured slower: it
            // costs registers and the masked body's extra work is small.)
            if (mcls != kSkip) tile(std::integral_constant<int, 2>{});
        } else if (R == 1 || on) {
            tile(std::integral_constant<int, VARIANT == kSigmoid ? 0 : 1>{});
        }

        if (nxt >= 0) stage.store(Ks[buf ^ 1], Vs[buf ^ 1]);
        if constexpr (MASKED)
            if (nxt >= 0) mcls = mstage.store(Ms[buf ^ 1], q0, nxt * BK, n, nxt_want);
        on = nxt_want != kWantNone;
        __syncthreads();
        buf ^= 1;
        kt = nxt;
    }

    // Finalise and store: oacc[mp][db][4i + j] is map mp's O^T entry for
    // O[qr][32 db + 8 i + 4 hh + j]; differential attention writes
    // O1 - lambda O2.
    float inv[MAPS];
#pragma unroll
    for (int mp = 0; mp < MAPS; ++mp) {
        inv[mp] = 1.0f;
        if (kSoft) {
            const float l_tot = l_run[mp] + __shfl_xor(l_run[mp], 32);
            inv[mp] = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if (lseb[mp] && hh == 0 && qr < L) {
                float lse = -INFINITY;
                if (q_valid && l_tot > 0.0f) lse = (m_run[mp] + __builtin_log2f(l_tot)) * kLn2;
                lseb[mp][qr] = lse;
            }
        }
    }
    if constexpr (MAPS == 2) {
        // Each map's own output, when asked for (the backward needs them).
        if (qr < L) {
#pragma unroll
            for (int mp = 0; mp < MAPS; ++mp) {
                bf16 *om = reinterpret_cast<bf16 *>(mp == 0 ? p.o1 : p.o2);
                if (om == nullptr) continue;
                bf16 *orow = om + b * p.osb + h * p.osh + (int64_t)qr * p.osl;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        auto f = [&](int e) { return keep_or_zero(oacc[mp][db][4 * i + e] * inv[mp], q_valid); };
                        *reinterpret_cast<bf16x4 *>(orow + db * 32 + i * 8 + hh * 4) =
                            pack4(f(0), f(1), f(2), f(3));
                    }
            }
        }
        inv[1] *= -p.lambda;
    }
    if (qr < L) {
        bf16 *orow = ob + (int64_t)qr * p.osl;
        // Padded query rows are exactly +0 whatever their (finite) accumulators hold.
        auto out = [&](int db, int e) {
            float x = oacc[0][db][e] * inv[0];
            if constexpr (MAPS == 2) x = fmaf(oacc[1][db][e], inv[1], x);
            return keep_or_zero(x, q_valid);
        };
        if constexpr (VARIANT == kDiffSecond) {
            // The second map of a two-pass differential forward: its own
            // output to o2 (when asked for), and o = O1 - lambda O2 with O1
            // the first pass's stored bf16 output (o1, which may be o itself:
            // each lane reads its elements before it writes them).
            const int64_t roff = b * p.osb + h * p.osh + (int64_t)qr * p.osl;
            const bf16 *o1row = reinterpret_cast<const bf16 *>(p.o1) + roff;
            bf16 *o2row = p.o2 != nullptr ? reinterpret_cast<bf16 *>(p.o2) + roff : nullptr;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = db * 32 + i * 8 + hh * 4;
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = out(db, 4 * i + e);
                    if (o2row != nullptr)
                        *reinterpret_cast<bf16x4 *>(o2row + col) = pack4(x[0], x[1], x[2], x[3]);
                    const bf16x4 first = *reinterpret_cast<const bf16x4 *>(o1row + col);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[e] = keep_or_zero(fmaf(-p.lambda, x[e], (float)first[e]), q_valid);
                    *reinterpret_cast<bf16x4 *>(orow + col) = pack4(x[0], x[1], x[2], x[3]);
                }
        } else {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bf16x4 v4 = pack4(out(db, 4 * i), out(db, 4 * i + 1),
                                            out(db, 4 * i + 2), out(db, 4 * i + 3));
                    *reinterpret_cast<bf16x4 *>(orow + db * 32 + i * 8 + hh * 4) = v4;
                }
        }
    }
    // Without a schedule: this tile's share of the sequence's fully padded
    // query tiles, issued last: nothing waits for these stores (before the
    // loop, the first tile's wait for its loads also waited for them, since
    // stores count in vmcnt).
    if constexpr (!LIST) padded_share<BQ>(qt, n, L, zero_tile);
}

template <int D, int VARIANT>
hipError_t launch_fwd_d(const AttnParams &p, hipStream_t stream) {
    static_assert(VARIANT != kDiff || D == 64, "two maps in one loop at d = 64 only");
    constexpr int NW = 4, BQ = 32 * NW;
    const int rows = BQ / p.block_q;  // block-mask rows per workgroup: 1, 2 or 4
    // At d = 128 the forward visits 32 keys at a time: 64-key steps hold
    // about 210 VGPRs (two waves per SIMD), 32-key steps are held to 168
    // (three).
    const int kb = p.block_k >= 64 && D == 64 ? 2 : 1;
    const dim3 grid = tile_grid((p.L + BQ - 1) / BQ, p.B, p.H);
    dim3 block(64 * NW);
#define SIGATTN_FWD_LAUNCH(KB_, MASK_, R_)                                                         \
    if (p.items1 != nullptr)                                                                       \
        hipLaunchKernelGGL((fwd_kernel<D, VARIANT, NW, KB_, MASK_, R_, true>), grid, block, 0,     \
                           stream, p);                                                             \
    else                                                                                           \
        hipLaunchKernelGGL((fwd_kernel<D, VARIANT, NW, KB_, MASK_, R_, false>), grid, block, 0,    \
                           stream, p);
#define SIGATTN_FWD_CASE(R_, KB_)                                                                  \
    if constexpr (D == 64 || KB_ == 1)                                                             \
    if (rows == R_ && kb == KB_) {                                                                 \
        if (p.mask_bits != nullptr) { /* a dense mask, packed in the schedule */                  \
            hipLaunchKernelGGL((fwd_kernel<D, VARIANT, NW, KB_, kMaskBits, R_, true>), grid,      \
                               block, 0, stream, p);                                               \
        } else if (p.mask != nullptr) {                                                            \
            SIGATTN_FWD_LAUNCH(KB_, kMaskDense, R_)                                                \
        } else if (p.key_range != nullptr) {                                                       \
            SIGATTN_FWD_LAUNCH(KB_, kMaskRange, R_)                                                \
        } else {                                                                                   \
            SIGATTN_FWD_LAUNCH(KB_, kMaskNone, R_)                                                 \
        }                                                                                          \
        return hipGetLastError();                                                                  \
    }
    SIGATTN_FWD_CASE(1, 2)
    SIGATTN_FWD_CASE(1, 1)
    SIGATTN_FWD_CASE(2, 2)
    SIGATTN_FWD_CASE(2, 1)
    SIGATTN_FWD_CASE(4, 2)
    SIGATTN_FWD_CASE(4, 1)
#undef SIGATTN_FWD_CASE
#undef SIGATTN_FWD_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace sigattn
