// Forward kernel: fused, tiled attention over a padded variable-length batch
// for gfx950 (sigmoid, online softmax and softmax_1 through one tile loop).
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
//   S^T = K Q^T           32x32x16 bf16 MFMA, K from LDS, Q held in registers
//   P^T = f(S^T)          epilogue in registers (sigmoid, or online softmax)
//   O^T += V^T P^T        P^T stays in registers as the B operand; V^T comes
//                         from a transposed, key-permuted copy of V in LDS
// Computing the transposed products puts one query per lane (lane % 32), so
// softmax row statistics are lane-local plus one exchange with lane ^ 32.
// The next tile's K/V are fetched into registers while the current tile
// computes.  Fully padded query tiles only write zeros.
#include "device_common.h"
#include "kernels.h"

namespace sigattn {

namespace {

template <int D, int BK, int NT>
struct KVStage {
    // Each thread moves CH 16-byte chunks of K and of V per tile.
    static constexpr int kChunksPerRow = D / 8;
    static constexpr int CH = BK * kChunksPerRow / NT;
    static_assert(CH * NT == BK * kChunksPerRow, "tile must split evenly over threads");
    uint4 k[CH], v[CH];

    __device__ __forceinline__ void load(const bf16 *kb, const bf16 *vb, int64_t sl, int k0,
                                         int n, int tid) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            const int row = idx / kChunksPerRow, col = (idx % kChunksPerRow) * 8;
            const int key = k0 + row;
            if (key < n) {
                k[c] = load16(kb + (int64_t)key * sl + col);
                v[c] = load16(vb + (int64_t)key * sl + col);
            } else {
                k[c] = make_uint4(0, 0, 0, 0);
                v[c] = make_uint4(0, 0, 0, 0);
            }
        }
    }

    // K row-major [BK][D + 8]; V transposed [D][BK + 8] with keys in perm16 order.
    __device__ __forceinline__ void store(bf16 (*Ks)[D + 8], bf16 (*Vt)[BK + 8], int tid) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int idx = tid + c * NT;
            const int row = idx / kChunksPerRow, col = (idx % kChunksPerRow) * 8;
            *reinterpret_cast<uint4 *>(&Ks[row][col]) = k[c];
            const bf16x8 vv = as_bf16x8(v[c]);
            const int pos = perm16(row);
#pragma unroll
            for (int e = 0; e < 8; ++e) Vt[col + e][pos] = vv[e];
        }
    }
};

__device__ __forceinline__ bool tile_active(const uint8_t *bm_row, int k0, int block_k) {
    return bm_row == nullptr || bm_row[k0 / block_k] != 0;
}

}  // namespace

template <int D, int VARIANT, int NW, int KB>
__global__ void __launch_bounds__(64 * NW)
fwd_kernel(const AttnParams p) {
    constexpr int BQ = 32 * NW, BK = 32 * KB, NT = 64 * NW;
    constexpr int KS = D / 16;  // MFMA k-steps over the head dimension
    constexpr int DB = D / 32;  // 32-wide blocks of the head dimension
    __shared__ __attribute__((aligned(16))) bf16 Ks[BK][D + 8];
    __shared__ __attribute__((aligned(16))) bf16 Vt[D][BK + 8];

    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int L = p.L;
    const int n = clamp_len(p.seq_lens[b], L);
    const int q0 = qt * BQ;
    bf16 *ob = reinterpret_cast<bf16 *>(p.o) + b * p.osb + h * p.osh;
    float *lseb = p.lse ? p.lse + ((int64_t)b * p.H + h) * L : nullptr;

    if (q0 >= n) {  // fully padded query tile: zero rows, nothing else
        const int rows = min(BQ, L - q0);
        for (int idx = tid; idx < rows * (D / 8); idx += NT) {
            const int r = q0 + idx / (D / 8), c = (idx % (D / 8)) * 8;
            *reinterpret_cast<uint4 *>(ob + (int64_t)r * p.osl + c) = make_uint4(0, 0, 0, 0);
        }
        if (VARIANT != kSigmoid && lseb)
            for (int r = q0 + tid; r < q0 + rows; r += NT) lseb[r] = -INFINITY;
        return;
    }

    const bf16 *qb = reinterpret_cast<const bf16 *>(p.q) + b * p.sb + h * p.sh;
    const bf16 *kb = reinterpret_cast<const bf16 *>(p.k) + b * p.sb + h * p.sh;
    const bf16 *vb = reinterpret_cast<const bf16 *>(p.v) + b * p.sb + h * p.sh;
    const uint8_t *bm_row =
        p.block_mask ? p.block_mask + ((int64_t)b * p.Tq + q0 / p.block_q) * p.Tk : nullptr;
    const uint8_t *mrow = nullptr;

    const int ql = lane & 31, hh = lane >> 5;
    const int qr = q0 + w * 32 + ql;  // this lane's query row
    const bool q_valid = qr < n;
    if (p.mask && q_valid) mrow = p.mask + ((int64_t)b * L + qr) * L;

    // Q^T operand: lane holds Q[qr][16 ks + 8 hh .. + 7].
    bf16x8 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qreg[ks] = q_valid ? as_bf16x8(load16(qb + (int64_t)qr * p.sl + ks * 16 + hh * 8))
                           : as_bf16x8(make_uint4(0, 0, 0, 0));

    const float beta = bias_value(p.bias_mode, n, L);
    // SIGMOID: u = -(s) * log2 e; softmax: t = s * log2 e (log2-domain logits).
    const float c1 = VARIANT == kSigmoid ? -p.scale * kLog2e : p.scale * kLog2e;
    const float c0 = VARIANT == kSigmoid ? -beta * kLog2e : beta * kLog2e;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_run = VARIANT == kSoftmax1 ? 0.0f : -INFINITY;  // log2 domain
    float l_run = (VARIANT == kSoftmax1 && hh == 0) ? 1.0f : 0.0f;  // split over lane halves

    const int nkt = (n + BK - 1) / BK;
    int kt = 0;
    while (kt < nkt && !tile_active(bm_row, kt * BK, p.block_k)) ++kt;
    KVStage<D, BK, NT> stage;
    if (kt < nkt) stage.load(kb, vb, p.sl, kt * BK, n, tid);

    while (kt < nkt) {
        const int k0 = kt * BK;
        __syncthreads();
        stage.store(Ks, Vt, tid);
        __syncthreads();
        int nxt = kt + 1;
        while (nxt < nkt && !tile_active(bm_row, nxt * BK, p.block_k)) ++nxt;
        if (nxt < nkt) stage.load(kb, vb, p.sl, nxt * BK, n, tid);

        // S^T for each 32-key block of the tile.
        f32x16 sacc[KB];
#pragma unroll
        for (int kb2 = 0; kb2 < KB; ++kb2) {
            sacc[kb2] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a =
                    *reinterpret_cast<const bf16x8 *>(&Ks[kb2 * 32 + ql][ks * 16 + hh * 8]);
                sacc[kb2] = mfma32(a, qreg[ks], sacc[kb2]);
            }
        }

        // Validity: tile fully inside [0, n) x [0, n) and no element mask -> all valid.
        const bool full = (k0 + BK <= n) && (q0 + BQ <= n) && (p.mask == nullptr);
        float pv[KB][16];
        if (VARIANT == kSigmoid) {
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb2 * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
                    bool ok = full || (q_valid && key < n && (mrow == nullptr || mrow[key]));
                    pv[kb2][r] = ok ? sigmoid_from(sacc[kb2][r], c1, c0) : 0.0f;
                }
        } else {
            float tmax = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb2 * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
                    bool ok = full || (q_valid && key < n && (mrow == nullptr || mrow[key]));
                    const float t = ok ? fmaf(sacc[kb2][r], c1, c0) : -INFINITY;
                    pv[kb2][r] = t;
                    tmax = fmaxf(tmax, t);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = m_new == -INFINITY ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float psum = 0.0f;
#pragma unroll
            for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = __builtin_amdgcn_exp2f(pv[kb2][r] - m_use);
                    pv[kb2][r] = e;
                    psum += e;
                }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }

        // O^T += V^T P^T over the tile's 32-key blocks (two 16-key MFMA steps each).
#pragma unroll
        for (int kb2 = 0; kb2 < KB; ++kb2) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 pb = pack8(&pv[kb2][kk * 8]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        &Vt[db * 32 + ql][kb2 * 32 + kk * 16 + hh * 8]);
                    oacc[db] = mfma32(a, pb, oacc[db]);
                }
            }
        }
        kt = nxt;
    }

    // Finalise and store: oacc[db][4i + j] is O[qr][32 db + 8 i + 4 hh + j].
    float inv = 1.0f;
    if (VARIANT != kSigmoid) {
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if (lseb && hh == 0 && qr < L) {
            float lse = -INFINITY;
            if (q_valid && l_tot > 0.0f) lse = (m_run + __builtin_log2f(l_tot)) * kLn2;
            lseb[qr] = lse;
        }
    }
    if (qr < L) {
        bf16 *orow = ob + (int64_t)qr * p.osl;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x16 &a = oacc[db];
                const bf16x4 v4 = pack4(a[4 * i] * inv, a[4 * i + 1] * inv, a[4 * i + 2] * inv,
                                        a[4 * i + 3] * inv);
                *reinterpret_cast<bf16x4 *>(orow + db * 32 + i * 8 + hh * 4) = v4;
            }
    }
}

template <int D, int VARIANT>
static hipError_t launch_fwd_d(const AttnParams &p, hipStream_t stream) {
    const int nw = p.block_q >= 128 ? 4 : p.block_q / 32;
    const int kb = p.block_k >= 64 ? 2 : 1;
    const int bq = 32 * nw;
    dim3 grid((p.L + bq - 1) / bq, p.H, p.B);
    dim3 block(64 * nw);
#define SIGATTN_FWD_CASE(NW_, KB_)                                                        \
    if (nw == NW_ && kb == KB_) {                                                         \
        hipLaunchKernelGGL((fwd_kernel<D, VARIANT, NW_, KB_>), grid, block, 0, stream, p); \
        return hipGetLastError();                                                         \
    }
    SIGATTN_FWD_CASE(4, 2)
    SIGATTN_FWD_CASE(4, 1)
    SIGATTN_FWD_CASE(2, 2)
    SIGATTN_FWD_CASE(2, 1)
    SIGATTN_FWD_CASE(1, 2)
    SIGATTN_FWD_CASE(1, 1)
#undef SIGATTN_FWD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_fwd(const AttnParams &p, hipStream_t stream) {
    if (p.d == 64) {
        if (p.variant == kSigmoid) return launch_fwd_d<64, kSigmoid>(p, stream);
        if (p.variant == kSoftmax) return launch_fwd_d<64, kSoftmax>(p, stream);
        return launch_fwd_d<64, kSoftmax1>(p, stream);
    }
    if (p.variant == kSigmoid) return launch_fwd_d<128, kSigmoid>(p, stream);
    if (p.variant == kSoftmax) return launch_fwd_d<128, kSoftmax>(p, stream);
    return launch_fwd_d<128, kSoftmax1>(p, stream);
}

}  // namespace sigattn
