// Backward kernel templates (included by one translation unit per variant):
// the backward pass on gfx950 (sigmoid, and the softmax variants from the
// forward's LSE): dK/dV work items and dQ work items (each kind its own
// kernel, or both in one grid), no atomics, scores and weights recomputed on
// the fly
// ("Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", section 2.C).  The Jacobian of element-wise sigmoid
// attention is diagonal (section 2.B), so with P = sigma(S) and
// dP = dO V^T the score gradient is dS = dP * P * (1 - P), element by element.
//
// dK/dV item: a workgroup of NW waves owns 32*NW keys of one (batch entry,
// head); each wave holds its 32 K rows in registers, and its V rows in
// registers (d = 64) or LDS (d = 128), and walks the query tiles whose
// block-mask entry is non-zero (one column of the block matrix):
//   S  = Q K^T,  dP = dO V^T            (Q, dO rows from LDS)
//   dV^T += dO^T P,  dK^T += Q^T dS     (P, dS stay in registers; Q^T and dO^T
//                                        come from transposing LDS reads)
// dQ item: a workgroup owns 32*NW queries; each wave holds its Q and dO rows
// and walks the key tiles of one block-mask row:
//   S^T = K Q^T,  dP^T = V dO^T         (K, V rows from LDS)
//   dQ^T += K^T dS^T                    (K^T from transposing LDS reads)
// Tiles are double-buffered in LDS (unpadded, XOR-swizzled rows) with one
// barrier per tile; the next tile is fetched through bounds-checked buffer
// loads while the current one computes -- into registers for dK/dV, straight
// into LDS for dQ (its K and V buffers are separate LDS objects and its loop
// is unrolled by two, so the compiler sees the buffer being filled is not the
// one being read; the freed staging registers let S and dP keep separate
// accumulators).  The two kinds of item write disjoint outputs.  Element
// masks arrive per tile as LDS bits, as in the forward kernel.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace sigattn {

namespace {

// Moves a [BT x D] tile of two tensors (rows [r0, n) of each; rows >= n read
// as zeros) into swizzled LDS tiles, CH 16-byte chunks per thread and tensor.
template <int D, int BT, int NT>
struct PairStage {
    static constexpr int kChunksPerRow = D / 8;
    static constexpr int CH = BT * kChunksPerRow / NT;
    static_assert(CH * NT == BT * kChunksPerRow, "tile must split evenly over threads");
    uint4 a[CH], b[CH];
    int goff[CH], loff[CH];

    __device__ __forceinline__ void init(int64_t sl, int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            const int row = idx / kChunksPerRow, col = (idx % kChunksPerRow) * 8;
            goff[c] = (int)(((int64_t)row * sl + col) * 2);
            loff[c] = swz_off<D>(row, col);
        }
    }

    __device__ __forceinline__ void load(rsrc_t ra, rsrc_t rb) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            a[c] = buffer_load16(ra, goff[c]);
            b[c] = buffer_load16(rb, goff[c]);
        }
    }

    __device__ __forceinline__ void store(bf16 *ta, bf16 *tb) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            *reinterpret_cast<uint4 *>(ta + loff[c]) = a[c];
            *reinterpret_cast<uint4 *>(tb + loff[c]) = b[c];
        }
    }
};

// A third tensor of the same tile shape, moved with a PairStage's offsets.
template <int D, int BT, int NT>
struct OneStage {
    static constexpr int CH = PairStage<D, BT, NT>::CH;
    uint4 a[CH];

    __device__ __forceinline__ void load(rsrc_t ra, const int (&goff)[CH]) {
#pragma unroll
        for (int c = 0; c < CH; ++c) a[c] = buffer_load16(ra, goff[c]);
    }

    __device__ __forceinline__ void store(bf16 *ta, const int (&loff)[CH]) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) *reinterpret_cast<uint4 *>(ta + loff[c]) = a[c];
    }
};

// Fetches a [BT x D] tile of two tensors straight into swizzled LDS tiles
// (buffer loads that write LDS, no staging registers).  One wave
// instruction fills one contiguous KiB, lane l the 16 bytes at 16 l, so each
// lane reads the global 16-byte chunk that the XOR swizzle (swz_off) places
// at its slot.  Rows >= n read as zeros through the descriptor.
template <int D, int BT, int NW>
struct DmaPair {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kBlocks = BT * kRowBytes / 1024;  // KiB blocks per tile
    static constexpr int kPerWave = kBlocks / NW;
    static_assert(kPerWave * NW == kBlocks, "tile must split evenly over the waves");
    int goff[kPerWave];
    int lds_off;  // byte offset of this wave's first block inside a tile

    __device__ __forceinline__ void init(int64_t sl, int w, int lane) {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const int byte = (w * kPerWave + i) * 1024 + lane * 16;
            const int row = byte / kRowBytes, pos = (byte % kRowBytes) / 16;
            goff[i] = (int)(((int64_t)row * sl + (pos ^ swz(row)) * 8) * 2);
        }
        lds_off = w * kPerWave * 1024;
    }

    __device__ __forceinline__ void issue(rsrc_t ra, rsrc_t rb, bf16 *ta, bf16 *tb) const {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            lds_load16(ra, reinterpret_cast<char *>(ta) + lds_off + i * 1024, goff[i]);
            lds_load16(rb, reinterpret_cast<char *>(tb) + lds_off + i * 1024, goff[i]);
        }
    }

    // A third tensor of the same tile shape.
    __device__ __forceinline__ void issue_one(rsrc_t ra, bf16 *ta) const {
#pragma unroll
        for (int i = 0; i < kPerWave; ++i)
            lds_load16(ra, reinterpret_cast<char *>(ta) + lds_off + i * 1024, goff[i]);
    }
};

// Dot product of two rows of eight bf16 values, accumulated in fp32.
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
    const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc = fmaf(__uint_as_float(x[i] << 16), __uint_as_float(y[i] << 16), acc);
        acc = fmaf(__uint_as_float(x[i] & 0xffff0000u), __uint_as_float(y[i] & 0xffff0000u), acc);
    }
    return acc;
}

// Softmax-family backward, dK/dV side: per query row of a staged tile, the
// weight offset off = b log2 e - lse log2 e (-inf for a row without weights:
// padded, or no valid key) and D = rowsum(dO * O).  D comes from the dO
// chunks a PairStage holds and an O tile fetched alongside with the same
// chunk-to-thread map; the lanes that hold one row are consecutive, so a
// short xor reduction finishes each row.
template <int D, int BT, int NT>
struct RowStats {
    static constexpr int kChunksPerRow = D / 8;
    static constexpr int CH = BT * kChunksPerRow / NT;
    uint4 o[CH];
    int goff[CH];
    float lse;

    __device__ __forceinline__ void init(int64_t osl, int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            goff[c] = (int)(((int64_t)(idx / kChunksPerRow) * osl + (idx % kChunksPerRow) * 8) * 2);
        }
    }

    // O rows [r0, n) through ro; lse_rows points at the LSE of row r0.
    __device__ __forceinline__ void load(rsrc_t ro, const float *lse_rows, int valid_rows,
                                         int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) o[c] = buffer_load16(ro, goff[c]);
        lse = (tid < BT && tid < valid_rows) ? lse_rows[tid] : -INFINITY;
    }

    __device__ __forceinline__ void store(const uint4 *dout_chunks, float c0, float *d_lds,
                                          float *off_lds, int tid) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const float part = group_sum<kChunksPerRow>(dot8(dout_chunks[c], o[c]));
            const int idx = tid + c * NT;
            if (idx % kChunksPerRow == 0) d_lds[idx / kChunksPerRow] = part;
        }
        if (tid < BT) off_lds[tid] = lse == -INFINITY ? -INFINITY : c0 - lse * kLog2e;
    }
};

template <int D>
__device__ __forceinline__ void zero_rows(bf16 *base, int64_t sl, int r0, int rows, int tid,
                                          int nt) {
    for (int idx = tid; idx < rows * (D / 8); idx += nt) {
        const int r = r0 + idx / (D / 8), c = (idx % (D / 8)) * 8;
        *reinterpret_cast<uint4 *>(base + (int64_t)r * sl + c) = make_uint4(0, 0, 0, 0);
    }
}

// acc[db][4i + j] holds X^T[32 db + 8 i + 4 hh + j][row]; store scale * X[row][:],
// or exact zeros for a padded row.  accumulate: add to what a previous launch
// stored.  lo_rowp (or null): the row of a second bf16 tensor for the
// rounding residual, written (x - bf16(x)) without accumulate and added back
// with it.
template <int D>
__device__ __forceinline__ void store_rows_t(bf16 *rowp, const f32x16 *acc, float scale, int hh,
                                             bool row_valid, bool accumulate = false,
                                             bf16 *lo_rowp = nullptr) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = db * 32 + i * 8 + hh * 4;
            bf16x4 *dst = reinterpret_cast<bf16x4 *>(rowp + col);
            bf16x4 *lo = lo_rowp != nullptr ? reinterpret_cast<bf16x4 *>(lo_rowp + col) : nullptr;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = acc[db][4 * i + e] * scale;
            if (accumulate) {  // a second pass adds to what the first wrote
                const bf16x4 old = *dst;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] += (float)old[e];
                if (lo != nullptr) {
                    const bf16x4 old_lo = *lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] += (float)old_lo[e];
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = keep_or_zero(x[e], row_valid);
            const bf16x4 hi = pack4(x[0], x[1], x[2], x[3]);
            *dst = hi;
            if (lo != nullptr && !accumulate)
                *lo = pack4(x[0] - (float)hi[0], x[1] - (float)hi[1], x[2] - (float)hi[2],
                            x[3] - (float)hi[3]);
        }
}

// 16-byte row operand of a swizzled tile: row r, columns [col, col + 8).
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const bf16 *tile, int r, int col) {
    return *reinterpret_cast<const bf16x8 *>(tile + swz_off<D>(r, col));
}

// Transposed operand of a swizzled tile for a 16-row MFMA step starting at
// row r16: lane gets column `col` (its lane % 32 within the 32-column block
// starting at c32) at rows r16 + {4h+j, 8+4h+j}.  trow / tcol as in fwd.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const bf16 *tile, int r16, int c32, int trow,
                                             int tcol) {
    const int r = r16 + trow;
    return cat8(lds_read_tr4(tile + swz_off<D>(r, c32 + tcol)),
                lds_read_tr4(tile + swz_off<D>(r + 8, c32 + tcol)));
}

}  // namespace

// ---------------------------------------------------------------- dK / dV
// Softmax maps per work item: two for differential attention (both maps'
// gradients in one pass: dP = dO V^T serves both, and dV takes the combined
// weights P1 - lambda P2), one otherwise.
template <int VARIANT> constexpr int kMapsOf = VARIANT == kDiff ? 2 : 1;

// LDS of one dK/dV tile (elements): Q (per map) and dO tiles of 32 rows,
// double-buffered, then two buffers of MAPS x 2 x 32 floats of row statistics
// (softmax variants).
template <int D, int MAPS = 1>
constexpr int kDkdvLds = (MAPS + 1) * 2 * 32 * D + 2 * MAPS * 2 * 32 * 2;

// Element-mask bits of two tiles (MaskStage words), for either kind of work.
constexpr int kMaskWords = 2 * 256;

// At d = 128, and with two maps, the V rows of a wave's keys wait in LDS
// (32 x D elements per wave) rather than in registers: the dK and dV
// accumulators and the K rows leave too few registers for the tile loop
// otherwise.
template <int D, int VARIANT> constexpr bool kVInLds = D == 128 || VARIANT == kDiff;

// dK and dV of key tile kt (32 NW keys) of (batch entry b, head h); smem
// holds kDkdvLds<D, MAPS> elements, mbits kMaskWords words (element mask
// only), vt this wave's 32 x D elements when kVInLds<D, VARIANT>.  Differential
// attention (two maps): also dK2, with S2 = Q2 K2^T, dS2 = P2 (dP - D2) and
// dK2 = -lambda scale dS2^T Q2, and dV from the weights P1 - lambda P2.
// C: block-mask columns per workgroup (BKV / block_k); wave w follows column
// w * C / NW and works only on the query tiles that column keeps.
template <int D, int NW, int VARIANT, int MASK, int C, bool LIST>
__device__ __forceinline__ void dkdv_tile(const AttnParams &p, int b, int h, int kt, int n,
                                          bf16 *smem, uint32_t *mbits, bf16 *vt) {
    constexpr bool MASKED = MASK != kMaskNone;
    constexpr int BKV = 32 * NW, BQ = 32, NT = 64 * NW;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr bool kSoft = VARIANT != kSigmoid;
    constexpr int MAPS = kMapsOf<VARIANT>;
    // Slot i of the Q and dO tiles (and map 2's Q) and of map mp's row
    // statistics (offsets from the LDS base, so the LDS address space stays
    // visible to the compiler).
    auto Qs = [&](int i) { return smem + i * (BQ * D); };
    auto dOs = [&](int i) { return smem + (2 + i) * (BQ * D); };
    auto Q2s = [&](int i) { return smem + (4 + i) * (BQ * D); };
    auto Dl = [&](int i, int mp = 0) {
        return reinterpret_cast<float *>(smem + 2 * (MAPS + 1) * BQ * D) + (i * MAPS + mp) * 2 * BQ;
    };
    auto Offl = [&](int i, int mp = 0) { return Dl(i, mp) + BQ; };

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int L = p.L;
    const int k0 = kt * BKV;
    bf16 *dkb = reinterpret_cast<bf16 *>(p.dk) + b * p.osb + h * p.osh;
    bf16 *dvb = reinterpret_cast<bf16 *>(p.dv) + b * p.osb + h * p.osh;
    bf16 *dk2b = MAPS == 2 ? reinterpret_cast<bf16 *>(p.dk2) + b * p.osb + h * p.osh : nullptr;
    auto zero_tile = [&](int r0, int rows) {
        zero_rows<D>(dkb, p.osl, r0, rows, tid, NT);
        zero_rows<D>(dvb, p.osl, r0, rows, tid, NT);
        if constexpr (MAPS == 2) zero_rows<D>(dk2b, p.osl, r0, rows, tid, NT);
    };
    if (k0 >= n) {  // a zero item: zeros, nothing else
        zero_tile(k0, zero_item_rows<BKV, LIST>(k0, L));
        return;
    }
    const bf16 *qb = reinterpret_cast<const bf16 *>(p.q) + b * p.sb + h * p.sh;
    const bf16 *kb = reinterpret_cast<const bf16 *>(p.k) + b * p.sb + h * p.sh;
    const bf16 *vb = reinterpret_cast<const bf16 *>(p.v) + b * p.sb + h * p.sh;
    const bf16 *dob = reinterpret_cast<const bf16 *>(p.dout) + b * p.sb + h * p.sh;
    const bf16 *obase = kSoft ? reinterpret_cast<const bf16 *>(p.o) + b * p.osb + h * p.osh
                              : nullptr;
    const float *lseb = kSoft ? p.lse + ((int64_t)b * p.H + h) * L : nullptr;
    const bf16 *qb2 = nullptr, *k2base = nullptr, *obase2 = nullptr;
    const float *lseb2 = nullptr;
    if constexpr (MAPS == 2) {
        qb2 = reinterpret_cast<const bf16 *>(p.q2) + b * p.sb + h * p.sh;
        k2base = reinterpret_cast<const bf16 *>(p.k2) + b * p.sb + h * p.sh;
        obase2 = reinterpret_cast<const bf16 *>(p.o2) + b * p.osb + h * p.osh;
        lseb2 = p.lse2 + ((int64_t)b * p.H + h) * L;
    }

    const int kl = lane & 31, hh = lane >> 5;
    const int key = k0 + w * 32 + kl;  // this lane's key row
    const bool k_valid = key < n;
    const int trow = 4 * hh + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const MaskSource msrc = mask_source<MASK>(p, b);
    // Mask words: key kl of this wave's 32 is one bit of the word of each query row.
    const int mbit = key_bit<MASK>(kl);
    using Mask = MaskStager<MASK, BQ, BKV, NT, false>;
    int mcls = kMixed;  // this wave's 32 x 32 entries of the current tile
    auto Ml = [&](int i) { return mbits + i * Mask::kWords; };

    // K^T and V^T operands of S = Q K^T and dP = dO V^T: lane holds row `key`.
    const rsrc_t rk = make_rsrc(kb + (int64_t)k0 * p.sl, (int64_t)(n - k0) * p.sl * 2);
    const rsrc_t rv = make_rsrc(vb + (int64_t)k0 * p.sl, (int64_t)(n - k0) * p.sl * 2);
    constexpr bool kVLds = kVInLds<D, VARIANT>;
    bf16x8 kreg[KS], vreg[kVLds ? 1 : KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int off = (int)(((int64_t)(w * 32 + kl) * p.sl + ks * 16 + hh * 8) * 2);
        kreg[ks] = as_bf16x8(buffer_load16(rk, off));
        const uint4 v8 = buffer_load16(rv, off);
        // Each lane reads back only the 16 bytes it wrote (swizzled like the
        // Q tile, so the reads spread over the banks).
        if constexpr (kVLds)
            *reinterpret_cast<uint4 *>(vt + swz_off<D>(kl, ks * 16 + hh * 8)) = v8;
        else
            vreg[ks] = as_bf16x8(v8);
    }
    auto v_operand = [&](int ks) {
        if constexpr (kVLds)
            return row_operand<D>(vt, kl, ks * 16 + hh * 8);
        else
            return vreg[ks];
    };
    bf16x8 kreg2[MAPS == 2 ? KS : 1];
    if constexpr (MAPS == 2) {
        const rsrc_t rk2 = make_rsrc(k2base + (int64_t)k0 * p.sl, (int64_t)(n - k0) * p.sl * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kreg2[ks] = as_bf16x8(buffer_load16(
                rk2, (int)(((int64_t)(w * 32 + kl) * p.sl + ks * 16 + hh * 8) * 2)));
    }
    // SIGMOID: K is scaled by c1 before the loop, so the S accumulator is
    // u = -scale * s * log2 e (see sigmoid_scaled).  Softmax: the weight is
    // exp2(s * c1 + off) with c1 = scale * log2 e and off from RowStats.
    const float c1 = kSoft ? p.scale * kLog2e : -p.scale * kLog2e;
    const float cexp = bias_factor(p.bias_mode, n, L);
    const float c0 = bias_value(p.bias_mode, n, L) * kLog2e;

    f32x16 dvt[DB], dkt[DB], dkt2[MAPS == 2 ? DB : 1];
#pragma unroll
    for (int db = 0; db < DB; ++db) dvt[db] = dkt[db] = f32x16{};
    if constexpr (MAPS == 2)
#pragma unroll
        for (int db = 0; db < DB; ++db) dkt2[db] = f32x16{};

    auto rows_rsrc = [&](const bf16 *base, int r0) {
        return make_rsrc(base + (int64_t)r0 * p.sl, (int64_t)(n - r0) * p.sl * 2);
    };
    auto out_rows_rsrc = [&](const bf16 *base, int r0) {
        return make_rsrc(base + (int64_t)r0 * p.osl, (int64_t)(n - r0) * p.osl * 2);
    };
    PairStage<D, BQ, NT> stage;
    stage.init(p.sl, tid);
    OneStage<D, BQ, NT> stage2;  // map 2's Q
    RowStats<D, BQ, NT> stats, stats2;
    if constexpr (kSoft) stats.init(p.osl, tid);
    if constexpr (MAPS == 2) stats2.init(p.osl, tid);
    Mask mstage;
    if constexpr (MASKED) mstage.init(tid);
    // want: what this wave needs of the tile's element mask (kWant*).
    auto load_tile = [&](int t, int want) {
        stage.load(rows_rsrc(qb, t * BQ), rows_rsrc(dob, t * BQ));
        if constexpr (MAPS == 2) stage2.load(rows_rsrc(qb2, t * BQ), stage.goff);
        if constexpr (kSoft) stats.load(out_rows_rsrc(obase, t * BQ), lseb + t * BQ, n - t * BQ, tid);
        if constexpr (MAPS == 2)
            stats2.load(out_rows_rsrc(obase2, t * BQ), lseb2 + t * BQ, n - t * BQ, tid);
        if constexpr (MASKED) mstage.load(msrc, n, t * BQ, k0, want);
    };
    auto store_tile = [&](int i, int t, int want) {
        stage.store(Qs(i), dOs(i));
        if constexpr (MAPS == 2) stage2.store(Q2s(i), stage.loff);
        if constexpr (kSoft) stats.store(stage.b, c0, Dl(i), Offl(i), tid);
        if constexpr (MAPS == 2) stats2.store(stage.b, c0, Dl(i, 1), Offl(i, 1), tid);
        if constexpr (MASKED) mcls = mstage.store(Ml(i), t * BQ, k0, n, want);
    };
    // Query tile 0 is fetched before the block mask is read (see the forward
    // kernel); another first tile is fetched again.
    load_tile(0, kWantMask);
    const int line0 = k0 / p.block_k;  // first block-mask column of this tile
    const int wl = w * C / NW;        // this wave's column (0 .. C - 1)
    const int lines = p.block_mask ? min(C, p.Tk - line0)
                                   : min(C, (n - k0 + p.block_k - 1) / p.block_k);
    Schedule<BQ, C, false, LIST> sched;
    if constexpr (LIST)
        sched.init(p.klist + ((int64_t)b * ((L + 127) / 128) + kt) * p.kstride, p.Tq, wl, n,
                   p.block_q);
    else
        sched.init(p.block_mask ? p.block_mask + (int64_t)b * p.Tq * p.Tk + line0 : nullptr,
                   p.Tk, lines, wl, n, p.block_q);
    int qt = sched.next();
    const int qt_want = sched.want();
    bool on = qt_want != kWantNone;  // this wave's column keeps the current tile
    if (qt > 0) load_tile(qt, qt_want);
    int buf = 0;
    store_tile(0, qt < 0 ? 0 : qt, qt_want);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        if constexpr (!kSoft) kreg[ks] = scale8(kreg[ks], c1);
    __syncthreads();

    while (qt >= 0) {
        const int nxt = sched.next();
        const int nxt_want = sched.want();
        if (nxt >= 0) load_tile(nxt, nxt_want);
        const bf16 *Qc = Qs(buf);
        const bf16 *dOc = dOs(buf);
        const float *Dc = Dl(buf);
        const float *Offc = Offl(buf);
        const bf16 *Q2c = Q2s(buf);
        const float *D2c = Dl(buf, MAPS - 1);
        const float *Off2c = Offl(buf, MAPS - 1);
        const uint32_t *Mc = Ml(buf);
        // One body per tile kind (its only branch is the uniform one around
        // the element-mask selects).  MODE 0 (no element mask)
        // needs no per-element masking: padded query rows of Q and dO read as
        // zeros, so dP = 0 and dS = 0 there (softmax: their off is -inf, so
        // P = 0) and their dV terms multiply zero rows; padded key rows are
        // zeroed at the store.  MODE 2: element mask.
        auto tile = [&](auto mode_tag) {
            constexpr int MODE = decltype(mode_tag)::value;
            f32x16 s = f32x16{}, dp = f32x16{}, s2 = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s = mfma32(row_operand<D>(Qc, kl, ks * 16 + hh * 8), kreg[ks], s);
                dp = mfma32(row_operand<D>(dOc, kl, ks * 16 + hh * 8), v_operand(ks), dp);
                if constexpr (MAPS == 2)
                    s2 = mfma32(row_operand<D>(Q2c, kl, ks * 16 + hh * 8), kreg2[ks], s2);
            }
            // s[4i + j] = S[query q0 + 8 i + 4 hh + j][key]
            // MODE 2: mask words of query rows 8 i + 4 hh + j (validity folded
            // in), read and applied only when this wave's share of the tile
            // is not entirely kept (a uniform branch): masked scores turn into
            // the values whose weights are exactly 0.
            if constexpr (MODE == 2) {
                if (mcls != kDense) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint4 m4 = *reinterpret_cast<const uint4 *>(Mc + w * 32 + 8 * i + 4 * hh);
                        s[4 * i + 0] = keep_score<kSoft>(s[4 * i + 0], mask_select(m4.x, mbit));
                        s[4 * i + 1] = keep_score<kSoft>(s[4 * i + 1], mask_select(m4.y, mbit));
                        s[4 * i + 2] = keep_score<kSoft>(s[4 * i + 2], mask_select(m4.z, mbit));
                        s[4 * i + 3] = keep_score<kSoft>(s[4 * i + 3], mask_select(m4.w, mbit));
                        if constexpr (MAPS == 2) {
                            s2[4 * i + 0] = keep_score<kSoft>(s2[4 * i + 0], mask_select(m4.x, mbit));
                            s2[4 * i + 1] = keep_score<kSoft>(s2[4 * i + 1], mask_select(m4.y, mbit));
                            s2[4 * i + 2] = keep_score<kSoft>(s2[4 * i + 2], mask_select(m4.z, mbit));
                            s2[4 * i + 3] = keep_score<kSoft>(s2[4 * i + 3], mask_select(m4.w, mbit));
                        }
                    }
                }
            }
            float pv[16], dsv[16], dsv2[MAPS == 2 ? 16 : 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // Softmax row statistics of query rows 8 i + 4 hh + j, read
                // four rows at a time (all sixteen at once cost registers).
                f32x4 offq, dq4, offq2, dq42;
                if constexpr (kSoft) {
                    offq = *reinterpret_cast<const f32x4 *>(Offc + 8 * i + 4 * hh);
                    dq4 = *reinterpret_cast<const f32x4 *>(Dc + 8 * i + 4 * hh);
                }
                if constexpr (MAPS == 2) {
                    offq2 = *reinterpret_cast<const f32x4 *>(Off2c + 8 * i + 4 * hh);
                    dq42 = *reinterpret_cast<const f32x4 *>(D2c + 8 * i + 4 * hh);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * i + j;
                    float pr;
                    if constexpr (kSoft)
                        pr = __builtin_amdgcn_exp2f(fmaf(s[r], c1, offq[j]));
                    else
                        pr = sigmoid_scaled(s[r], cexp);
                    pv[r] = pr;
                    if constexpr (kSoft)
                        dsv[r] = pr * (dp[r] - dq4[j]);
                    else
                        dsv[r] = dp[r] * (pr - pr * pr);
                    if constexpr (MAPS == 2) {
                        // Map 2's score gradient without its factor -lambda
                        // (applied at the dK2 store); dV's weight P1 - lambda P2.
                        const float pr2 = __builtin_amdgcn_exp2f(fmaf(s2[r], c1, offq2[j]));
                        dsv2[r] = pr2 * (dp[r] - dq42[j]);
                        pv[r] = fmaf(-p.lambda, pr2, pr);
                    }
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 pb = pack8(&pv[kk * 8]);
                const bf16x8 sb = pack8(&dsv[kk * 8]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    dvt[db] = mfma32(tr_operand<D>(dOc, kk * 16, db * 32, trow, tcol), pb, dvt[db]);
                    dkt[db] = mfma32(tr_operand<D>(Qc, kk * 16, db * 32, trow, tcol), sb, dkt[db]);
                }
                if constexpr (MAPS == 2) {
                    const bf16x8 sb2 = pack8(&dsv2[kk * 8]);
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        dkt2[db] = mfma32(tr_operand<D>(Q2c, kk * 16, db * 32, trow, tcol), sb2,
                                          dkt2[db]);
                }
            }
        };
        if constexpr (MASKED) {
            // This wave's 32 x 32 entries, as found when it staged them: none
            // kept means no work.
            if (mcls != kSkip) tile(std::integral_constant<int, 2>{});
        } else if (C == 1 || on) {
            tile(std::integral_constant<int, 0>{});
        }
        if (nxt >= 0) store_tile(buf ^ 1, nxt, nxt_want);
        on = nxt_want != kWantNone;
        __syncthreads();
        buf ^= 1;
        qt = nxt;
    }
    if (key < L) {
        // The dv residual's row is read (with accumulate_dv) before this
        // lane's own dk store: the one tensor may serve as both (a
        // two-launch sum parks the residual in the second launch's dk).
        bf16 *lo = p.dv_lo != nullptr ? reinterpret_cast<bf16 *>(p.dv_lo) + b * p.osb +
                                            h * p.osh + (int64_t)key * p.osl
                                      : nullptr;
        store_rows_t<D>(dvb + (int64_t)key * p.osl, dvt, p.grad_scale, hh, k_valid,
                        p.accumulate_dv != 0, lo);
        store_rows_t<D>(dkb + (int64_t)key * p.osl, dkt, p.scale * p.grad_scale, hh, k_valid);
        if constexpr (MAPS == 2)
            store_rows_t<D>(dk2b + (int64_t)key * p.osl, dkt2, -p.lambda * p.scale * p.grad_scale,
                            hh, k_valid);
    }
    // Without a schedule: this tile's share of the sequence's fully padded
    // key tiles, issued last (nothing waits for these stores).
    if constexpr (!LIST) padded_share<BKV>(kt, n, L, zero_tile);
}

// ---------------------------------------------------------------- dQ
// dQ of query tile qt (32 NW queries) of (batch entry b, head h), visiting
// keys 32 KB at a time.  K0, V0, K1, V1 are four separate LDS objects of
// 32 KB rows x D each (two buffers of the K and V tiles); with two maps
// (differential attention) K20, K21 are the two buffers of map 2's K tile,
// and dQ2 = -lambda scale dS2 K2 is computed beside dQ.
// R: block-mask rows per workgroup (BQ / block_q); wave w follows row
// w * R / NW.
template <int D, int NW, int KB, int VARIANT, int MASK, int R, bool LIST>
__device__ __forceinline__ void dq_tile(const AttnParams &p, int b, int h, int qt, int n,
                                        bf16 *K0, bf16 *V0, bf16 *K1, bf16 *V1,
                                        uint32_t *mbits, bf16 *K20 = nullptr,
                                        bf16 *K21 = nullptr) {
    constexpr bool MASKED = MASK != kMaskNone;
    constexpr int BQ = 32 * NW, BK = 32 * KB, NT = 64 * NW;
    constexpr int KS = D / 16, DB = D / 32;
    constexpr bool kSoft = VARIANT != kSigmoid;
    constexpr int MAPS = kMapsOf<VARIANT>;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = p.L;
    const int q0 = qt * BQ;
    bf16 *dqb = reinterpret_cast<bf16 *>(p.dq) + b * p.osb + h * p.osh;
    bf16 *dq2b = MAPS == 2 ? reinterpret_cast<bf16 *>(p.dq2) + b * p.osb + h * p.osh : nullptr;
    auto zero_tile = [&](int r0, int rows) {
        zero_rows<D>(dqb, p.osl, r0, rows, tid, NT);
        if constexpr (MAPS == 2) zero_rows<D>(dq2b, p.osl, r0, rows, tid, NT);
    };
    if (q0 >= n) {  // a zero item: zeros, nothing else
        zero_tile(q0, zero_item_rows<BQ, LIST>(q0, L));
        return;
    }
    const bf16 *qb = reinterpret_cast<const bf16 *>(p.q) + b * p.sb + h * p.sh;
    const bf16 *kb = reinterpret_cast<const bf16 *>(p.k) + b * p.sb + h * p.sh;
    const bf16 *vb = reinterpret_cast<const bf16 *>(p.v) + b * p.sb + h * p.sh;
    const bf16 *dob = reinterpret_cast<const bf16 *>(p.dout) + b * p.sb + h * p.sh;

    const int ql = lane & 31, hh = lane >> 5;
    const int qr = q0 + w * 32 + ql;
    const bool q_valid = qr < n;
    const int trow = 4 * hh + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const MaskSource msrc = mask_source<MASK>(p, b);
    using Mask = MaskStager<MASK, BQ, BK, NT, true>;
    int mcls = kMixed;  // this wave's share of the current tile
    uint32_t *M0 = mbits, *M1 = mbits + Mask::kWords;

    const rsrc_t rq = make_rsrc(qb + (int64_t)q0 * p.sl, (int64_t)(n - q0) * p.sl * 2);
    const rsrc_t rdo = make_rsrc(dob + (int64_t)q0 * p.sl, (int64_t)(n - q0) * p.sl * 2);
    bf16x8 qreg[KS], doreg[KS], qreg2[MAPS == 2 ? KS : 1];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int off = (int)(((int64_t)(w * 32 + ql) * p.sl + ks * 16 + hh * 8) * 2);
        qreg[ks] = as_bf16x8(buffer_load16(rq, off));
        doreg[ks] = as_bf16x8(buffer_load16(rdo, off));
    }
    const bf16 *k2base = nullptr;
    if constexpr (MAPS == 2) {
        const bf16 *qb2 = reinterpret_cast<const bf16 *>(p.q2) + b * p.sb + h * p.sh;
        k2base = reinterpret_cast<const bf16 *>(p.k2) + b * p.sb + h * p.sh;
        const rsrc_t rq2 = make_rsrc(qb2 + (int64_t)q0 * p.sl, (int64_t)(n - q0) * p.sl * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qreg2[ks] = as_bf16x8(buffer_load16(
                rq2, (int)(((int64_t)(w * 32 + ql) * p.sl + ks * 16 + hh * 8) * 2)));
    }
    // SIGMOID: Q is scaled by c1 before the loop, so the S accumulator is
    // u = -scale * s * log2 e (see sigmoid_scaled).  Softmax: the weight is
    // exp2(s * c1 + off) with c1 = scale * log2 e, off = b log2 e - lse log2 e
    // (-inf for a padded row or one without weights), and dS = P (dP - D)
    // with D = rowsum(dO * O) of this lane's query.
    const float c1 = kSoft ? p.scale * kLog2e : -p.scale * kLog2e;
    const float cexp = bias_factor(p.bias_mode, n, L);
    float off = 0.0f, drow = 0.0f;
    if constexpr (kSoft) {
        const bf16 *ob = reinterpret_cast<const bf16 *>(p.o) + b * p.osb + h * p.osh;
        const rsrc_t ro = make_rsrc(ob + (int64_t)q0 * p.osl, (int64_t)(n - q0) * p.osl * 2);
        float part = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 o8 = buffer_load16(
                ro, (int)(((int64_t)(w * 32 + ql) * p.osl + ks * 16 + hh * 8) * 2));
            part += dot8(__builtin_bit_cast(uint4, doreg[ks]), o8);
        }
        drow = part + __shfl_xor(part, 32);
        const float lse = q_valid ? p.lse[((int64_t)b * p.H + h) * L + qr] : -INFINITY;
        off = lse == -INFINITY ? -INFINITY
                               : bias_value(p.bias_mode, n, L) * kLog2e - lse * kLog2e;
    }
    // Map 2's row statistics, from its own output O2 and LSE.
    float off2 = 0.0f, drow2 = 0.0f;
    if constexpr (MAPS == 2) {
        const bf16 *ob2 = reinterpret_cast<const bf16 *>(p.o2) + b * p.osb + h * p.osh;
        const rsrc_t ro2 = make_rsrc(ob2 + (int64_t)q0 * p.osl, (int64_t)(n - q0) * p.osl * 2);
        float part = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 o8 = buffer_load16(
                ro2, (int)(((int64_t)(w * 32 + ql) * p.osl + ks * 16 + hh * 8) * 2));
            part += dot8(__builtin_bit_cast(uint4, doreg[ks]), o8);
        }
        drow2 = part + __shfl_xor(part, 32);
        const float lse2 = q_valid ? p.lse2[((int64_t)b * p.H + h) * L + qr] : -INFINITY;
        off2 = lse2 == -INFINITY ? -INFINITY
                                 : bias_value(p.bias_mode, n, L) * kLog2e - lse2 * kLog2e;
    }

    f32x16 dqt[DB], dqt2[MAPS == 2 ? DB : 1];
#pragma unroll
    for (int db = 0; db < DB; ++db) dqt[db] = f32x16{};
    if constexpr (MAPS == 2)
#pragma unroll
        for (int db = 0; db < DB; ++db) dqt2[db] = f32x16{};

    auto rows_rsrc = [&](const bf16 *base, int r0) {
        return make_rsrc(base + (int64_t)r0 * p.sl, (int64_t)(n - r0) * p.sl * 2);
    };
    // Key tile 0 is fetched before the block mask is read (see the forward
    // kernel); another first tile is fetched again.  Tiles go straight into
    // LDS; the two buffers are separate LDS objects and the loop below is
    // unrolled by two, so the compiler sees that the buffer being filled is
    // not the one being read.
    DmaPair<D, BK, NW> dma;
    dma.init(p.sl, w, lane);
    auto fetch = [&](int t, bf16 *kd, bf16 *vd, bf16 *k2d) {
        dma.issue(rows_rsrc(kb, t * BK), rows_rsrc(vb, t * BK), kd, vd);
        if constexpr (MAPS == 2) dma.issue_one(rows_rsrc(k2base, t * BK), k2d);
    };
    fetch(0, K0, V0, K20);
    Mask mstage;
    if constexpr (MASKED) mstage.init(tid);
    const int line0 = q0 / p.block_q;  // first block-mask row of this tile
    const int wl = w * R / NW;        // this wave's row (0 .. R - 1)
    const int lines = p.block_mask ? min(R, p.Tq - line0)
                                   : min(R, (n - q0 + p.block_q - 1) / p.block_q);
    Schedule<BK, R, true, LIST> sched;
    if constexpr (LIST)
        sched.init(p.qlist + ((int64_t)b * ((L + 127) / 128) + qt) * p.qstride, p.Tk, wl, n,
                   p.block_k);
    else
        sched.init(p.block_mask ? p.block_mask + ((int64_t)b * p.Tq + line0) * p.Tk : nullptr,
                   p.Tk, lines, wl, n, p.block_k);
    int kt = sched.next();
    const int kt_want = sched.want();
    bool on = kt_want != kWantNone;  // this wave's row keeps the current tile
    if (kt > 0) fetch(kt, K0, V0, K20);
    if constexpr (MASKED)
        if (kt >= 0) {
            mstage.load(msrc, n, q0, kt * BK, kt_want);
            mcls = mstage.store(M0, q0, kt * BK, n, kt_want);
        }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        if constexpr (!kSoft) qreg[ks] = scale8(qreg[ks], c1);
    wait_vm0();
    __syncthreads();

    auto step = [&](const bf16 *Kc, const bf16 *Vc, const uint32_t *Mc, bf16 *Kn, bf16 *Vn,
                    uint32_t *Mn, const bf16 *K2c, bf16 *K2n) {
        const int nxt = sched.next();
        const int nxt_want = sched.want();
        if (nxt >= 0) fetch(nxt, Kn, Vn, K2n);
        if constexpr (MASKED)
            if (nxt >= 0) mstage.load(msrc, n, q0, nxt * BK, nxt_want);
        // MODE 0 (no element mask): padded key rows of K and V read as zeros,
        // so dP = 0 and dS = 0 there; padded query rows are zeroed at the
        // store.  MODE 2: element mask.
        auto tile = [&](auto mode_tag) {
            constexpr int MODE = decltype(mode_tag)::value;
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2) {
                f32x16 s = f32x16{}, dp = f32x16{}, s2 = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s = mfma32(row_operand<D>(Kc, kb2 * 32 + ql, ks * 16 + hh * 8), qreg[ks], s);
                    dp = mfma32(row_operand<D>(Vc, kb2 * 32 + ql, ks * 16 + hh * 8), doreg[ks],
                                dp);
                    if constexpr (MAPS == 2)
                        s2 = mfma32(row_operand<D>(K2c, kb2 * 32 + ql, ks * 16 + hh * 8),
                                    qreg2[ks], s2);
                }
                // s[4i + j] = S^T[key k0 + 32 kb2 + 8 i + 4 hh + j][qr]; in
                // MODE 2 that key is bit key_bit(8 i + 4 hh + j) of the row's
                // mask word: 8 j + 2 i + hh (dense) or 8 i + 4 hh + j (ranges).
                constexpr bool kDenseBits = MASK == kMaskDense;
                // Applied only when this wave's share of the tile is not
                // entirely kept (a uniform branch).
                if constexpr (MODE == 2) {
                    if (mcls != kDense) {
                        const uint32_t mwk = Mc[kb2 * BQ + w * 32 + ql] >> (kDenseBits ? hh : 4 * hh);
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            s[r] = keep_score<kSoft>(
                                s[r], mask_select(mwk, kDenseBits ? 8 * (r & 3) + 2 * (r >> 2)
                                                                  : 8 * (r >> 2) + (r & 3)));
                        if constexpr (MAPS == 2)
#pragma unroll
                            for (int r = 0; r < 16; ++r)
                                s2[r] = keep_score<kSoft>(
                                    s2[r], mask_select(mwk, kDenseBits ? 8 * (r & 3) + 2 * (r >> 2)
                                                                       : 8 * (r >> 2) + (r & 3)));
                    }
                }
                float dsv[16], dsv2[MAPS == 2 ? 16 : 1];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float pr;
                    if constexpr (kSoft)
                        pr = __builtin_amdgcn_exp2f(fmaf(s[r], c1, off));
                    else
                        pr = sigmoid_scaled(s[r], cexp);
                    if constexpr (kSoft)
                        dsv[r] = pr * (dp[r] - drow);
                    else
                        dsv[r] = dp[r] * (pr - pr * pr);
                    if constexpr (MAPS == 2)  // without its factor -lambda
                        dsv2[r] = __builtin_amdgcn_exp2f(fmaf(s2[r], c1, off2)) * (dp[r] - drow2);
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 sb = pack8(&dsv[kk * 8]);
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        dqt[db] = mfma32(tr_operand<D>(Kc, kb2 * 32 + kk * 16, db * 32, trow, tcol),
                                         sb, dqt[db]);
                    if constexpr (MAPS == 2) {
                        const bf16x8 sb2 = pack8(&dsv2[kk * 8]);
#pragma unroll
                        for (int db = 0; db < DB; ++db)
                            dqt2[db] = mfma32(
                                tr_operand<D>(K2c, kb2 * 32 + kk * 16, db * 32, trow, tcol), sb2,
                                dqt2[db]);
                    }
                }
            }
        };
        if constexpr (MASKED) {
            // The wave's entries of this tile, as found when it staged them:
            // none kept means no work.
            if (mcls != kSkip) tile(std::integral_constant<int, 2>{});
        } else if (R == 1 || on) {
            tile(std::integral_constant<int, 0>{});
        }
        if constexpr (MASKED)
            if (nxt >= 0) mcls = mstage.store(Mn, q0, nxt * BK, n, nxt_want);
        on = nxt_want != kWantNone;
        wait_vm0();
        __syncthreads();
        kt = nxt;
    };
    while (kt >= 0) {
        step(K0, V0, M0, K1, V1, M1, K20, K21);
        if (kt < 0) break;
        step(K1, V1, M1, K0, V0, M0, K21, K20);
    }
    if (qr < L) {
        store_rows_t<D>(dqb + (int64_t)qr * p.osl, dqt, p.scale * p.grad_scale, hh, q_valid);
        if constexpr (MAPS == 2)
            store_rows_t<D>(dq2b + (int64_t)qr * p.osl, dqt2, -p.lambda * p.scale * p.grad_scale,
                            hh, q_valid);
    }
    // Without a schedule: this tile's share of the sequence's fully padded
    // query tiles, issued last (nothing waits for these stores).
    if constexpr (!LIST) padded_share<BQ>(qt, n, L, zero_tile);
}

// ---------------------------------------------------------------- kernels
// Waves per SIMD the register allocation must allow.  The unmasked kernels
// at d = 64 need about 168 VGPRs (the softmax variants a few more, spilled),
// and so does sigmoid with key ranges or a packed mask: held to that, three
// waves share a SIMD (LDS allows three workgroups per CU even in the
// one-launch kernel), 12 to 13 % faster than two.  The other masked kernels
// would spill more (76 to 152 bytes per lane) and gain nothing.
// Two maps (differential attention) hold twice the operands and accumulators:
// two waves.
template <int D, int VARIANT, int MASK>
constexpr int kBwdWavesPerSimd =
    D == 64 && VARIANT != kDiff && (MASK == kMaskNone ||
                (VARIANT == kSigmoid && (MASK == kMaskRange || MASK == kMaskBits)))
        ? 3
        : 2;

// LIST: built for a schedule (work items and kept-entry lists from it).
template <int D, int NW, int VARIANT, int MASK, int C, bool LIST>
__global__ void __launch_bounds__(64 * NW, (kBwdWavesPerSimd<D, VARIANT, MASK>))
bwd_dkdv_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) bf16 smem[kDkdvLds<D, kMapsOf<VARIANT>>];
    __shared__ __attribute__((aligned(16))) uint32_t mbits[MASK != kMaskNone ? kMaskWords : 1];
    __shared__ __attribute__((aligned(16))) bf16 vts[kVInLds<D, VARIANT> ? NW * 32 * D : 1];
    static_assert(32 * NW == 128, "work items are 128-row tiles");
    int b, h, kind, kt, n;
    if (!work_item<1, LIST>(p, b, h, kind, kt, n)) return;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    dkdv_tile<D, NW, VARIANT, MASK, C, LIST>(p, b, h, kt, n, smem, mbits, vts + w * 32 * D);
}

template <int D, int NW, int KB, int VARIANT, int MASK, int R, bool LIST>
__global__ void __launch_bounds__(64 * NW, (kBwdWavesPerSimd<D, VARIANT, MASK>))
bwd_dq_kernel(const AttnParams p) {
    constexpr int kTile = 32 * KB * D;
    constexpr int kTile2 = kMapsOf<VARIANT> == 2 ? kTile : 8;  // map 2's K buffers
    __shared__ __attribute__((aligned(1024))) bf16 K0[kTile], V0[kTile], K1[kTile], V1[kTile];
    __shared__ __attribute__((aligned(1024))) bf16 K20[kTile2], K21[kTile2];
    __shared__ __attribute__((aligned(16))) uint32_t mbits[MASK != kMaskNone ? kMaskWords : 1];
    static_assert(32 * NW == 128, "work items are 128-row tiles");
    int b, h, kind, qt, n;
    if (!work_item<1, LIST>(p, b, h, kind, qt, n)) return;
    dq_tile<D, NW, KB, VARIANT, MASK, R, LIST>(p, b, h, qt, n, K0, V0, K1, V1, mbits, K20, K21);
}

// dK/dV and dQ in one launch: both kinds of tile of a (batch entry, head)
// pair are dealt out together, longest sequences first, so the two share one
// ramp-up and one tail.  Needs the same 32 NW rows for the key tiles of
// dK/dV and the query tiles of dQ.
// R: block-mask rows and columns per workgroup (block_q == block_k).
template <int D, int NW, int KB, int VARIANT, int MASK, int R, bool LIST>
__global__ void __launch_bounds__(64 * NW, (kBwdWavesPerSimd<D, VARIANT, MASK>))
bwd_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) bf16 smem[kDkdvLds<D, kMapsOf<VARIANT>>];
    constexpr int kTile = 32 * KB * D;
    constexpr int kTile2 = kMapsOf<VARIANT> == 2 ? kTile : 8;  // map 2's K buffers
    __shared__ __attribute__((aligned(1024))) bf16 K0[kTile], V0[kTile], K1[kTile], V1[kTile];
    __shared__ __attribute__((aligned(1024))) bf16 K20[kTile2], K21[kTile2];
    __shared__ __attribute__((aligned(16))) uint32_t mbits[MASK != kMaskNone ? kMaskWords : 1];
    static_assert(32 * NW == 128, "work items are 128-row tiles");
    int b, h, kind, t, n;
    if (!work_item<2, LIST>(p, b, h, kind, t, n)) return;
    if (kind == 0) {
        // A workgroup does one kind of work: the dQ key buffers, each 32 KB
        // rows x D, hold the dK/dV waves' V rows (32 rows each).
        static_assert(!kVInLds<D, VARIANT> || NW <= 4, "V rows need one dQ buffer per wave");
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        bf16 *vt = w == 0 ? K0 : w == 1 ? V0 : w == 2 ? K1 : V1;
        dkdv_tile<D, NW, VARIANT, MASK, R, LIST>(p, b, h, t, n, smem, mbits, vt);
    }
    else
        dq_tile<D, NW, KB, VARIANT, MASK, R, LIST>(p, b, h, t, n, K0, V0, K1, V1, mbits, K20,
                                                   K21);
}

// Every workgroup runs four waves: 128 keys (dK/dV) or 128 queries (dQ), the
// block-mask columns or rows those cover (1, 2 or 4) given as a template
// argument.  dQ visits keys 32 KB at a time with 32 KB dividing block_k.
constexpr int kBwdWaves = 4;
static int dkdv_cols(const AttnParams &p) { return 32 * kBwdWaves / p.block_k; }
static int dq_rows(const AttnParams &p) { return 32 * kBwdWaves / p.block_q; }
// At d = 128, and with two maps, the dQ step visits 32 keys: with two 32-key
// blocks its S, dP and operand registers no longer fit without spilling
// (the 64-key forms are not built for them).
static int dq_key_blocks(const AttnParams &p) {
    return p.block_k >= 64 && p.d == 64 && p.variant != kDiff ? 2 : 1;
}

// Launches kernel template K<..., LIST> with LIST = (the call has a schedule).
#define SIGATTN_LIST_LAUNCH(KERNEL, ...)                                                           \
    if (p.items1 != nullptr)                                                                       \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, true>), grid, block, 0, stream, p);                \
    else                                                                                           \
        hipLaunchKernelGGL((KERNEL<__VA_ARGS__, false>), grid, block, 0, stream, p);

template <int D, int VARIANT>
hipError_t launch_dkdv_d(const AttnParams &p, hipStream_t stream) {
    constexpr int NW = kBwdWaves;
    const int cols = dkdv_cols(p);
    const dim3 grid = tile_grid((p.L + 32 * NW - 1) / (32 * NW), p.B, p.H);
    dim3 block(64 * NW);
#define SIGATTN_DKDV_CASE(C_)                                                                  \
    if (cols == C_) {                                                                          \
        if (p.mask != nullptr) {                                                               \
            if (p.mask_bits != nullptr) {                                                  \
                hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, VARIANT, kMaskBits, C_, true>), grid, \
                                   block, 0, stream, p);                                   \
            } else {                                                                   \
                hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, VARIANT, kMaskDense, C_, false>),    \
                                   grid, block, 0, stream, p);                             \
            }               \
        } else if (p.key_range != nullptr) {                                                   \
            SIGATTN_LIST_LAUNCH(bwd_dkdv_kernel, D, NW, VARIANT, kMaskRange, C_)               \
        } else {                                                                               \
            SIGATTN_LIST_LAUNCH(bwd_dkdv_kernel, D, NW, VARIANT, kMaskNone, C_)                \
        }                                                                                      \
        return hipGetLastError();                                                              \
    }
    SIGATTN_DKDV_CASE(1)
    SIGATTN_DKDV_CASE(2)
    SIGATTN_DKDV_CASE(4)
#undef SIGATTN_DKDV_CASE
    return hipErrorInvalidValue;
}

template <int D, int VARIANT>
hipError_t launch_dq_d(const AttnParams &p, hipStream_t stream) {
    constexpr int NW = kBwdWaves;
    const int rows = dq_rows(p), kb = dq_key_blocks(p);
    const dim3 grid = tile_grid((p.L + 32 * NW - 1) / (32 * NW), p.B, p.H);
    dim3 block(64 * NW);
#define SIGATTN_DQ_CASE(R_, KB_)                                                                 \
    if constexpr ((D == 64 && VARIANT != kDiff) || KB_ == 1)                                   \
    if (rows == R_ && kb == KB_) {                                                               \
        if (p.mask != nullptr) {                                                                 \
            if (p.mask_bits != nullptr) {                                                  \
                hipLaunchKernelGGL((bwd_dq_kernel<D, NW, KB_, VARIANT, kMaskBits, R_, true>),   \
                                   grid, block, 0, stream, p);                             \
            } else {                                                                   \
                hipLaunchKernelGGL((bwd_dq_kernel<D, NW, KB_, VARIANT, kMaskDense, R_, false>), \
                                   grid, block, 0, stream, p);                             \
            }              \
        } else if (p.key_range != nullptr) {                                                     \
            SIGATTN_LIST_LAUNCH(bwd_dq_kernel, D, NW, KB_, VARIANT, kMaskRange, R_)              \
        } else {                                                                                 \
            SIGATTN_LIST_LAUNCH(bwd_dq_kernel, D, NW, KB_, VARIANT, kMaskNone, R_)               \
        }                                                                                        \
        return hipGetLastError();                                                                \
    }
    SIGATTN_DQ_CASE(1, 2)
    SIGATTN_DQ_CASE(1, 1)
    SIGATTN_DQ_CASE(2, 2)
    SIGATTN_DQ_CASE(2, 1)
    SIGATTN_DQ_CASE(4, 2)
    SIGATTN_DQ_CASE(4, 1)
#undef SIGATTN_DQ_CASE
    return hipErrorInvalidValue;
}

template <int D, int VARIANT>
hipError_t launch_bwd_d(const AttnParams &p, hipStream_t stream) {
    constexpr int NW = kBwdWaves;
    const int lines = dq_rows(p), kb = dq_key_blocks(p);
    if (lines != dkdv_cols(p)) {  // block_q != block_k: two launches
        hipError_t e = launch_dkdv_d<D, VARIANT>(p, stream);
        return e != hipSuccess ? e : launch_dq_d<D, VARIANT>(p, stream);
    }
    const dim3 grid = tile_grid(2 * ((p.L + 32 * NW - 1) / (32 * NW)), p.B, p.H);
    dim3 block(64 * NW);
#define SIGATTN_BWD_CASE(R_, KB_)                                                              \
    if constexpr ((D == 64 && VARIANT != kDiff) || KB_ == 1)                                 \
    if (lines == R_ && kb == KB_) {                                                            \
        if (p.mask != nullptr) {                                                               \
            if (p.mask_bits != nullptr) {                                                  \
                hipLaunchKernelGGL((bwd_kernel<D, NW, KB_, VARIANT, kMaskBits, R_, true>),      \
                                   grid, block, 0, stream, p);                             \
            } else {                                                                   \
                hipLaunchKernelGGL((bwd_kernel<D, NW, KB_, VARIANT, kMaskDense, R_, false>),    \
                                   grid, block, 0, stream, p);                             \
            }               \
        } else if (p.key_range != nullptr) {                                                   \
            SIGATTN_LIST_LAUNCH(bwd_kernel, D, NW, KB_, VARIANT, kMaskRange, R_)               \
        } else {                                                                               \
            SIGATTN_LIST_LAUNCH(bwd_kernel, D, NW, KB_, VARIANT, kMaskNone, R_)                \
        }                                                                                      \
        return hipGetLastError();                                                              \
    }
    SIGATTN_BWD_CASE(1, 2)
    SIGATTN_BWD_CASE(1, 1)
    SIGATTN_BWD_CASE(2, 2)
    SIGATTN_BWD_CASE(2, 1)
    SIGATTN_BWD_CASE(4, 2)
    SIGATTN_BWD_CASE(4, 1)
#undef SIGATTN_BWD_CASE
    return hipErrorInvalidValue;
}

#undef SIGATTN_LIST_LAUNCH

}  // namespace sigattn
