// Backward kernels for sigmoid attention on gfx950: one kernel for dK/dV and
// one for dQ, no atomics, scores and weights recomputed on the fly
// ("Better Models, Faster Training: Sigmoid Attention for single-cell
// Foundation Models", section 2.C).  The Jacobian of element-wise sigmoid
// attention is diagonal (section 2.B), so with P = sigma(S) and
// dP = dO V^T the score gradient is dS = dP * P * (1 - P), element by element.
//
// dK/dV kernel: a workgroup of NW waves owns 32*NW keys of one (batch entry,
// head); each wave holds its 32 K and V rows in registers and walks the query
// tiles whose block-mask entry is 1 (one column of the block matrix):
//   S  = Q K^T,  dP = dO V^T            (Q, dO rows from LDS)
//   dV^T += dO^T P,  dK^T += Q^T dS     (P, dS stay in registers; Q^T, dO^T
//                                        from transposed, permuted LDS copies)
// dQ kernel: a workgroup owns 32*NW queries; each wave holds its Q and dO rows
// and walks the key tiles of one block-mask row:
//   S^T = K Q^T,  dP^T = V dO^T         (K, V rows from LDS)
//   dQ^T += K^T dS^T                    (K^T from a transposed LDS copy)
// The two kernels write disjoint outputs and are launched back to back on one
// stream.
#include "device_common.h"
#include "kernels.h"

namespace sigattn {

namespace {

// Stage a [BT x D] tile of one or two tensors: row-major copies [BT][D + 8]
// and, where requested, transposed copies [D][BT + 8] with rows in perm16 order.
template <int D, int BT, int NT>
struct TileStage {
    static constexpr int kChunksPerRow = D / 8;
    static constexpr int CH = BT * kChunksPerRow / NT;
    static_assert(CH * NT == BT * kChunksPerRow, "tile must split evenly over threads");
    uint4 a[CH], b[CH];

    __device__ __forceinline__ void load(const bf16 *pa, const bf16 *pb, int64_t sl, int r0,
                                         int n, int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            const int row = idx / kChunksPerRow, col = (idx % kChunksPerRow) * 8;
            const int r = r0 + row;
            if (r < n) {
                a[c] = load16(pa + (int64_t)r * sl + col);
                b[c] = load16(pb + (int64_t)r * sl + col);
            } else {
                a[c] = make_uint4(0, 0, 0, 0);
                b[c] = make_uint4(0, 0, 0, 0);
            }
        }
    }

    __device__ __forceinline__ static void put(const uint4 &x, bf16 (*rows)[D + 8],
                                               bf16 (*cols)[BT + 8], int idx) {
        const int row = idx / kChunksPerRow, col = (idx % kChunksPerRow) * 8;
        if (rows) *reinterpret_cast<uint4 *>(&rows[row][col]) = x;
        if (cols) {
            const bf16x8 xv = as_bf16x8(x);
            const int pos = perm16(row);
#pragma unroll
            for (int e = 0; e < 8; ++e) cols[col + e][pos] = xv[e];
        }
    }

    __device__ __forceinline__ void store(bf16 (*a_rows)[D + 8], bf16 (*a_cols)[BT + 8],
                                          bf16 (*b_rows)[D + 8], bf16 (*b_cols)[BT + 8],
                                          int tid) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            put(a[c], a_rows, a_cols, tid + c * NT);
            put(b[c], b_rows, b_cols, tid + c * NT);
        }
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

// acc[db][4i + j] holds X^T[32 db + 8 i + 4 hh + j][row]; store scale * X[row][:].
template <int D>
__device__ __forceinline__ void store_rows_t(bf16 *rowp, const f32x16 *acc, float scale, int hh) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x4 v4 = pack4(acc[db][4 * i] * scale, acc[db][4 * i + 1] * scale,
                                    acc[db][4 * i + 2] * scale, acc[db][4 * i + 3] * scale);
            *reinterpret_cast<bf16x4 *>(rowp + db * 32 + i * 8 + hh * 4) = v4;
        }
}

}  // namespace

// ---------------------------------------------------------------- dK / dV
template <int D, int NW, int QB>
__global__ void __launch_bounds__(64 * NW)
bwd_dkdv_kernel(const AttnParams p) {
    constexpr int BKV = 32 * NW, BQ = 32 * QB, NT = 64 * NW;
    constexpr int KS = D / 16, DB = D / 32;
    __shared__ __attribute__((aligned(16))) bf16 Qs[BQ][D + 8];
    __shared__ __attribute__((aligned(16))) bf16 Qt[D][BQ + 8];
    __shared__ __attribute__((aligned(16))) bf16 dOs[BQ][D + 8];
    __shared__ __attribute__((aligned(16))) bf16 dOt[D][BQ + 8];

    const int kt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int L = p.L;
    const int n = clamp_len(p.seq_lens[b], L);
    const int k0 = kt * BKV;
    bf16 *dkb = reinterpret_cast<bf16 *>(p.dk) + b * p.osb + h * p.osh;
    bf16 *dvb = reinterpret_cast<bf16 *>(p.dv) + b * p.osb + h * p.osh;
    if (k0 >= n) {
        const int rows = min(BKV, L - k0);
        zero_rows<D>(dkb, p.osl, k0, rows, tid, NT);
        zero_rows<D>(dvb, p.osl, k0, rows, tid, NT);
        return;
    }
    const bf16 *qb = reinterpret_cast<const bf16 *>(p.q) + b * p.sb + h * p.sh;
    const bf16 *kb = reinterpret_cast<const bf16 *>(p.k) + b * p.sb + h * p.sh;
    const bf16 *vb = reinterpret_cast<const bf16 *>(p.v) + b * p.sb + h * p.sh;
    const bf16 *dob = reinterpret_cast<const bf16 *>(p.dout) + b * p.sb + h * p.sh;

    const int kl = lane & 31, hh = lane >> 5;
    const int key = k0 + w * 32 + kl;  // this lane's key row
    const bool k_valid = key < n;
    // K^T and V^T operands of S = Q K^T and dP = dO V^T: lane holds row `key`.
    bf16x8 kreg[KS], vreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        kreg[ks] = as_bf16x8(k_valid ? load16(kb + (int64_t)key * p.sl + ks * 16 + hh * 8) : z);
        vreg[ks] = as_bf16x8(k_valid ? load16(vb + (int64_t)key * p.sl + ks * 16 + hh * 8) : z);
    }
    const float beta = bias_value(p.bias_mode, n, L);
    const float c1 = -p.scale * kLog2e, c0 = -beta * kLog2e;
    const int bj = k0 / p.block_k;

    f32x16 dvt[DB], dkt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dvt[db] = dkt[db] = f32x16{};

    const int nqt = (n + BQ - 1) / BQ;
    auto active = [&](int qt) {
        return p.block_mask == nullptr ||
               p.block_mask[((int64_t)b * p.Tq + (qt * BQ) / p.block_q) * p.Tk + bj] != 0;
    };
    int qt = 0;
    while (qt < nqt && !active(qt)) ++qt;
    TileStage<D, BQ, NT> stage;
    if (qt < nqt) stage.load(qb, dob, p.sl, qt * BQ, n, tid);

    while (qt < nqt) {
        const int q0 = qt * BQ;
        __syncthreads();
        stage.store(Qs, Qt, dOs, dOt, tid);
        __syncthreads();
        int nxt = qt + 1;
        while (nxt < nqt && !active(nxt)) ++nxt;
        if (nxt < nqt) stage.load(qb, dob, p.sl, nxt * BQ, n, tid);

        const bool full = (q0 + BQ <= n) && (k0 + BKV <= n) && (p.mask == nullptr);
#pragma unroll
        for (int qb2 = 0; qb2 < QB; ++qb2) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 aq =
                    *reinterpret_cast<const bf16x8 *>(&Qs[qb2 * 32 + kl][ks * 16 + hh * 8]);
                const bf16x8 ad =
                    *reinterpret_cast<const bf16x8 *>(&dOs[qb2 * 32 + kl][ks * 16 + hh * 8]);
                s = mfma32(aq, kreg[ks], s);
                dp = mfma32(ad, vreg[ks], dp);
            }
            // s[4i + j] = S[query q0 + 32 qb2 + 8 i + 4 hh + j][key]
            float pv[16], dsv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = q0 + qb2 * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
                bool ok = full || (k_valid && qr < n &&
                                   (p.mask == nullptr || p.mask[((int64_t)b * L + qr) * L + key]));
                const float pr = ok ? sigmoid_from(s[r], c1, c0) : 0.0f;
                pv[r] = pr;
                dsv[r] = dp[r] * pr * (1.0f - pr);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 pb = pack8(&pv[kk * 8]);
                const bf16x8 sb = pack8(&dsv[kk * 8]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 ado = *reinterpret_cast<const bf16x8 *>(
                        &dOt[db * 32 + kl][qb2 * 32 + kk * 16 + hh * 8]);
                    const bf16x8 aqt = *reinterpret_cast<const bf16x8 *>(
                        &Qt[db * 32 + kl][qb2 * 32 + kk * 16 + hh * 8]);
                    dvt[db] = mfma32(ado, pb, dvt[db]);
                    dkt[db] = mfma32(aqt, sb, dkt[db]);
                }
            }
        }
        qt = nxt;
    }
    if (key < L) {
        store_rows_t<D>(dvb + (int64_t)key * p.osl, dvt, 1.0f, hh);
        store_rows_t<D>(dkb + (int64_t)key * p.osl, dkt, p.scale, hh);
    }
}

// ---------------------------------------------------------------- dQ
template <int D, int NW, int KB>
__global__ void __launch_bounds__(64 * NW)
bwd_dq_kernel(const AttnParams p) {
    constexpr int BQ = 32 * NW, BK = 32 * KB, NT = 64 * NW;
    constexpr int KS = D / 16, DB = D / 32;
    __shared__ __attribute__((aligned(16))) bf16 Ks[BK][D + 8];
    __shared__ __attribute__((aligned(16))) bf16 Kt[D][BK + 8];
    __shared__ __attribute__((aligned(16))) bf16 Vs[BK][D + 8];

    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int L = p.L;
    const int n = clamp_len(p.seq_lens[b], L);
    const int q0 = qt * BQ;
    bf16 *dqb = reinterpret_cast<bf16 *>(p.dq) + b * p.osb + h * p.osh;
    if (q0 >= n) {
        zero_rows<D>(dqb, p.osl, q0, min(BQ, L - q0), tid, NT);
        return;
    }
    const bf16 *qb = reinterpret_cast<const bf16 *>(p.q) + b * p.sb + h * p.sh;
    const bf16 *kb = reinterpret_cast<const bf16 *>(p.k) + b * p.sb + h * p.sh;
    const bf16 *vb = reinterpret_cast<const bf16 *>(p.v) + b * p.sb + h * p.sh;
    const bf16 *dob = reinterpret_cast<const bf16 *>(p.dout) + b * p.sb + h * p.sh;

    const int ql = lane & 31, hh = lane >> 5;
    const int qr = q0 + w * 32 + ql;
    const bool q_valid = qr < n;
    bf16x8 qreg[KS], doreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const uint4 z = make_uint4(0, 0, 0, 0);
        qreg[ks] = as_bf16x8(q_valid ? load16(qb + (int64_t)qr * p.sl + ks * 16 + hh * 8) : z);
        doreg[ks] = as_bf16x8(q_valid ? load16(dob + (int64_t)qr * p.sl + ks * 16 + hh * 8) : z);
    }
    const uint8_t *mrow = (p.mask && q_valid) ? p.mask + ((int64_t)b * L + qr) * L : nullptr;
    const uint8_t *bm_row =
        p.block_mask ? p.block_mask + ((int64_t)b * p.Tq + q0 / p.block_q) * p.Tk : nullptr;
    const float beta = bias_value(p.bias_mode, n, L);
    const float c1 = -p.scale * kLog2e, c0 = -beta * kLog2e;

    f32x16 dqt[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dqt[db] = f32x16{};

    const int nkt = (n + BK - 1) / BK;
    auto active = [&](int t) { return bm_row == nullptr || bm_row[(t * BK) / p.block_k] != 0; };
    int kt = 0;
    while (kt < nkt && !active(kt)) ++kt;
    TileStage<D, BK, NT> stage;
    if (kt < nkt) stage.load(kb, vb, p.sl, kt * BK, n, tid);

    while (kt < nkt) {
        const int k0 = kt * BK;
        __syncthreads();
        stage.store(Ks, Kt, Vs, nullptr, tid);
        __syncthreads();
        int nxt = kt + 1;
        while (nxt < nkt && !active(nxt)) ++nxt;
        if (nxt < nkt) stage.load(kb, vb, p.sl, nxt * BK, n, tid);

        const bool full = (k0 + BK <= n) && (q0 + BQ <= n) && (p.mask == nullptr);
#pragma unroll
        for (int kb2 = 0; kb2 < KB; ++kb2) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ak =
                    *reinterpret_cast<const bf16x8 *>(&Ks[kb2 * 32 + ql][ks * 16 + hh * 8]);
                const bf16x8 av =
                    *reinterpret_cast<const bf16x8 *>(&Vs[kb2 * 32 + ql][ks * 16 + hh * 8]);
                s = mfma32(ak, qreg[ks], s);
                dp = mfma32(av, doreg[ks], dp);
            }
            // s[4i + j] = S^T[key k0 + 32 kb2 + 8 i + 4 hh + j][qr]
            float dsv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + kb2 * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
                bool ok = full || (q_valid && key < n && (mrow == nullptr || mrow[key]));
                const float pr = ok ? sigmoid_from(s[r], c1, c0) : 0.0f;
                dsv[r] = dp[r] * pr * (1.0f - pr);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 sb = pack8(&dsv[kk * 8]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 akt = *reinterpret_cast<const bf16x8 *>(
                        &Kt[db * 32 + ql][kb2 * 32 + kk * 16 + hh * 8]);
                    dqt[db] = mfma32(akt, sb, dqt[db]);
                }
            }
        }
        kt = nxt;
    }
    if (qr < L) store_rows_t<D>(dqb + (int64_t)qr * p.osl, dqt, p.scale, hh);
}

template <int D>
static hipError_t launch_dkdv_d(const AttnParams &p, hipStream_t stream) {
    // 32*NW keys per workgroup must divide block_k; 32*QB queries per step
    // must divide block_q.
    const int nw = p.block_k >= 128 ? 4 : p.block_k / 32;
    const int qb = p.block_q >= 64 ? 2 : 1;
    dim3 grid((p.L + 32 * nw - 1) / (32 * nw), p.H, p.B);
    dim3 block(64 * nw);
#define SIGATTN_DKDV_CASE(NW_, QB_)                                                     \
    if (nw == NW_ && qb == QB_) {                                                       \
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW_, QB_>), grid, block, 0, stream, p);  \
        return hipGetLastError();                                                       \
    }
    SIGATTN_DKDV_CASE(4, 2)
    SIGATTN_DKDV_CASE(4, 1)
    SIGATTN_DKDV_CASE(2, 2)
    SIGATTN_DKDV_CASE(2, 1)
    SIGATTN_DKDV_CASE(1, 2)
    SIGATTN_DKDV_CASE(1, 1)
#undef SIGATTN_DKDV_CASE
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_dq_d(const AttnParams &p, hipStream_t stream) {
    // 32*NW queries per workgroup must divide block_q; 32*KB keys per step
    // must divide block_k.
    const int nw = p.block_q >= 128 ? 4 : p.block_q / 32;
    const int kb = p.block_k >= 64 ? 2 : 1;
    dim3 grid((p.L + 32 * nw - 1) / (32 * nw), p.H, p.B);
    dim3 block(64 * nw);
#define SIGATTN_DQ_CASE(NW_, KB_)                                                     \
    if (nw == NW_ && kb == KB_) {                                                     \
        hipLaunchKernelGGL((bwd_dq_kernel<D, NW_, KB_>), grid, block, 0, stream, p);  \
        return hipGetLastError();                                                     \
    }
    SIGATTN_DQ_CASE(4, 2)
    SIGATTN_DQ_CASE(4, 1)
    SIGATTN_DQ_CASE(2, 2)
    SIGATTN_DQ_CASE(2, 1)
    SIGATTN_DQ_CASE(1, 2)
    SIGATTN_DQ_CASE(1, 1)
#undef SIGATTN_DQ_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv(const AttnParams &p, hipStream_t stream) {
    return p.d == 64 ? launch_dkdv_d<64>(p, stream) : launch_dkdv_d<128>(p, stream);
}

hipError_t launch_bwd_dq(const AttnParams &p, hipStream_t stream) {
    return p.d == 64 ? launch_dq_d<64>(p, stream) : launch_dq_d<128>(p, stream);
}

}  // namespace sigattn
