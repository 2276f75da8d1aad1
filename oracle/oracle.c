/*
 * CPU oracle for padded variable-length attention (sigmoid, softmax,
 * softmax_1), forward and backward, plus the binary block mask.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain statement of what
 * the GPU library must compute.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it; the GPU library never does, and the
 * two share no code.
 *
 * Inputs are bf16 bit patterns (uint16) widened exactly to the working type.
 * The file is compiled twice: REAL=double (suffix _f64, used for parity) and
 * REAL=float (suffix _f32, the fp32 statement of the same definitions).
 *
 * Definitions (per batch entry b and head h; n = clamp(seq_len, 0, L)):
 *   valid(r, c)  = r < n and c < n and (no mask or mask[r, c] != 0)
 *   beta         = 0 | -ln n | -ln L            (bias modes NONE / SEQLEN / PADLEN)
 *                  The -log(n) bias comes from "Sigmoid Attention for
 *                  single-cell Foundation Models", section 2.A.
 *   s[r, c]      = scale * <q_r, k_c> + beta   (scaled dot product, same page
 *                  and the standard-attention listing of the Flash Attention page)
 *   SIGMOID      p = 1 / (1 + exp(-s))          (single-cell page, section 2.A)
 *   SOFTMAX      p = exp(s - m) / sum exp(s - m), m = row max over valid keys
 *                  (Flash Attention page, "the mathematics": decomposition)
 *   SOFTMAX1     p = exp(s) / (1 + sum exp(s))  (softmax_1 / QuietAttention page,
 *                  "Proposition"), evaluated with m~ = max(0, row max)
 *   o_r          = sum_c p[r, c] v_c, and 0 for padded rows or rows without a
 *                  valid key
 *   lse_r        = log of the softmax denominator (m + ln l); -inf for padded
 *                  rows and for softmax rows without a valid key; unused for
 *                  SIGMOID (written as -inf)
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <tgmath.h>

#ifndef REAL
#define REAL double
#endif
#ifndef SFX
#define SFX _f64
#endif
#define CAT2(a, b) a##b
#define CAT(a, b) CAT2(a, b)
#define FN(name) CAT(name, SFX)

typedef REAL real;

enum { V_SIGMOID = 0, V_SOFTMAX = 1, V_SOFTMAX1 = 2 };
enum { B_NONE = 0, B_LOG_SEQLEN = 1, B_LOG_PADLEN = 2 };

static real widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (real)f;
}

static int clamp_len(int n, int L) { return n < 0 ? 0 : (n > L ? L : n); }

static real bias_value(int mode, int n, int L) {
    if (mode == B_LOG_SEQLEN) return -log((real)n);
    if (mode == B_LOG_PADLEN) return -log((real)L);
    return (real)0;
}

static int valid(int r, int c, int n, const uint8_t *mask, int L) {
    return r < n && c < n && (mask == NULL || mask[(size_t)r * L + c] != 0);
}

static real dot_bf16(const uint16_t *x, const uint16_t *y, int d) {
    real acc = 0;
    for (int t = 0; t < d; ++t) acc += widen(x[t]) * widen(y[t]);
    return acc;
}

static real score(const uint16_t *q, const uint16_t *k, int d, int r, int c, real scale, real beta) {
    return scale * dot_bf16(q + (size_t)r * d, k + (size_t)c * d, d) + beta;
}

static real sigmoid(real x) { return (real)1 / ((real)1 + exp(-x)); }

#ifdef ORACLE_WITH_BLOCKMASK
/*
 * Binary block mask ("Binary Block Masking", "Presentation" and "How it
 * works"): bit 0 of entry (b, i, j) is 1 when the tile rows
 * [i*bq, min((i+1)*bq, L)) x columns [j*bk, min((j+1)*bk, L)) hold at least
 * one valid element.  One matrix per batch entry, shared by every head.
 * Bit 1 marks a full tile (the same page's point that runs of non-zero blocks
 * need fewer checks, read as: a tile with every element valid needs no
 * per-element mask): the whole bq x bk tile lies inside [0, n) x [0, n) and
 * every element of it is valid.  Entries are therefore 0, 1 or 3.
 * seq_lens [B]; mask [B, L, L] or NULL; out [B, Tq, Tk].
 */
void oracle_blockmask(const int32_t *seq_lens, const uint8_t *mask, int B, int L, int bq, int bk,
                      uint8_t *out) {
    int Tq = (L + bq - 1) / bq, Tk = (L + bk - 1) / bk;
    for (int b = 0; b < B; ++b) {
        int n = clamp_len(seq_lens[b], L);
        const uint8_t *mb = mask ? mask + (size_t)b * L * L : NULL;
        for (int i = 0; i < Tq; ++i)
            for (int j = 0; j < Tk; ++j) {
                int any = 0;
                int all = (i + 1) * bq <= n && (j + 1) * bk <= n;
                for (int r = i * bq; r < (i + 1) * bq && r < L; ++r)
                    for (int c = j * bk; c < (j + 1) * bk && c < L; ++c) {
                        if (valid(r, c, n, mb, L))
                            any = 1;
                        else
                            all = 0;
                    }
                out[((size_t)b * Tq + i) * Tk + j] = (uint8_t)(any | (all << 1));
            }
    }
}
#endif

/*
 * Forward pass by the plain definition, one head, rows [r0, r1).
 * q, k, v: [L, d] bf16 bits, rows contiguous.  mask: [L, L] for this batch
 * entry or NULL.  o: [(r1 - r0), d].  lse: [(r1 - r0)].
 */
void FN(oracle_fwd_rows)(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const uint8_t *mask, int bias_mode, int variant,
                         real scale, int r0, int r1, real *o, real *lse) {
    int n = clamp_len(seq_len, L);
    real beta = n > 0 ? bias_value(bias_mode, n, L) : (real)0;
    real *s = (real *)malloc(sizeof(real) * (size_t)(L > 0 ? L : 1));
    char *ok = (char *)malloc((size_t)(L > 0 ? L : 1));
    for (int r = r0; r < r1; ++r) {
        real *orow = o + (size_t)(r - r0) * d;
        for (int t = 0; t < d; ++t) orow[t] = 0;
        lse[r - r0] = -INFINITY;
        if (r >= n) continue;
        int count = 0;
        real mx = -INFINITY;
        for (int c = 0; c < L; ++c) {
            ok[c] = (char)valid(r, c, n, mask, L);
            if (!ok[c]) continue;
            s[c] = score(q, k, d, r, c, scale, beta);
            if (s[c] > mx) mx = s[c];
            ++count;
        }
        if (variant == V_SIGMOID) {
            for (int c = 0; c < L; ++c) {
                if (!ok[c]) continue;
                real p = sigmoid(s[c]);
                for (int t = 0; t < d; ++t) orow[t] += p * widen(v[(size_t)c * d + t]);
            }
            continue;
        }
        /* SOFTMAX: exp(s - m) / sum; SOFTMAX1: the extra 1 is exp(0 - m~). */
        real m = mx;
        real denom = 0;
        if (variant == V_SOFTMAX1) {
            if (m < 0) m = 0;
            denom = exp(-m);
        } else if (count == 0) {
            continue; /* no valid key: output 0, lse -inf */
        }
        for (int c = 0; c < L; ++c)
            if (ok[c]) denom += exp(s[c] - m);
        for (int c = 0; c < L; ++c) {
            if (!ok[c]) continue;
            real p = exp(s[c] - m) / denom;
            for (int t = 0; t < d; ++t) orow[t] += p * widen(v[(size_t)c * d + t]);
        }
        lse[r - r0] = m + log(denom);
    }
    free(ok);
    free(s);
}

/*
 * Forward pass as the tiled algorithm, one head: query tiles of bq rows,
 * key tiles of bk columns visited in increasing order; a tile whose block
 * mask entry is 0 is skipped ("Binary Block Masking"; padded blocks skipped on
 * both sides in the single-cell page, section 2.C).  bm: [Tq, Tk] for this
 * batch entry, or NULL to visit every tile.
 *
 * Softmax variants keep the running maximum m, the running sum l and an
 * unnormalised accumulator per row, and merge each tile by rescaling with
 * exp(m_old - m_new) (Flash Attention page, "the mathematics": decomposition
 * and merge).  A tile with no valid element leaves the state untouched.
 * SOFTMAX starts from (m, l) = (-inf, 0); SOFTMAX1 from (0, 1), the zero
 * logit with a zero value that adds 1 to the denominator (softmax_1 page,
 * "Properties").  SIGMOID needs no state: each tile adds sigma(s) v.
 */
void FN(oracle_fwd_tiled)(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, const uint8_t *mask, const uint8_t *bm, int bq,
                          int bk, int bias_mode, int variant, real scale, real *o, real *lse) {
    int n = clamp_len(seq_len, L);
    real beta = n > 0 ? bias_value(bias_mode, n, L) : (real)0;
    int Tq = (L + bq - 1) / bq, Tk = (L + bk - 1) / bk;
    real *acc = (real *)malloc(sizeof(real) * (size_t)d);
    real *s = (real *)malloc(sizeof(real) * (size_t)bk);
    char *ok = (char *)malloc((size_t)bk);
    for (int i = 0; i < Tq; ++i) {
        for (int r = i * bq; r < (i + 1) * bq && r < L; ++r) {
            real m = variant == V_SOFTMAX1 ? (real)0 : -INFINITY;
            real l = variant == V_SOFTMAX1 ? (real)1 : (real)0;
            for (int t = 0; t < d; ++t) acc[t] = 0;
            for (int j = 0; j < Tk; ++j) {
                if (bm && !bm[(size_t)i * Tk + j]) continue;
                int c0 = j * bk, c1 = (j + 1) * bk < L ? (j + 1) * bk : L;
                real tmax = -INFINITY;
                for (int c = c0; c < c1; ++c) {
                    ok[c - c0] = (char)valid(r, c, n, mask, L);
                    if (!ok[c - c0]) continue;
                    s[c - c0] = score(q, k, d, r, c, scale, beta);
                    if (s[c - c0] > tmax) tmax = s[c - c0];
                }
                if (variant == V_SIGMOID) {
                    for (int c = c0; c < c1; ++c) {
                        if (!ok[c - c0]) continue;
                        real p = sigmoid(s[c - c0]);
                        for (int t = 0; t < d; ++t) acc[t] += p * widen(v[(size_t)c * d + t]);
                    }
                    continue;
                }
                real mnew = tmax > m ? tmax : m;
                if (mnew == -INFINITY) continue; /* nothing valid yet */
                real alpha = exp(m - mnew);
                l *= alpha;
                for (int t = 0; t < d; ++t) acc[t] *= alpha;
                for (int c = c0; c < c1; ++c) {
                    if (!ok[c - c0]) continue;
                    real e = exp(s[c - c0] - mnew);
                    l += e;
                    for (int t = 0; t < d; ++t) acc[t] += e * widen(v[(size_t)c * d + t]);
                }
                m = mnew;
            }
            real *orow = o + (size_t)r * d;
            lse[r] = -INFINITY;
            if (r >= n) {
                for (int t = 0; t < d; ++t) orow[t] = 0;
                continue;
            }
            if (variant == V_SIGMOID) {
                for (int t = 0; t < d; ++t) orow[t] = acc[t];
                continue;
            }
            if (l == 0) { /* softmax row with no valid key */
                for (int t = 0; t < d; ++t) orow[t] = 0;
                continue;
            }
            for (int t = 0; t < d; ++t) orow[t] = acc[t] / l;
            lse[r] = m + log(l);
        }
    }
    free(ok);
    free(s);
    free(acc);
}

/*
 * Row statistics needed by the softmax-family backward: for each query row
 * r < n, the shift m_r and denominator l_r, so that p[r, c] = exp(s - m_r) / l_r.
 */
static void row_stats(int L, int d, int n, const uint16_t *q, const uint16_t *k,
                      const uint8_t *mask, int variant, real scale, real beta, int r, real *m_out,
                      real *l_out) {
    real mx = -INFINITY;
    for (int c = 0; c < n; ++c)
        if (valid(r, c, n, mask, L)) {
            real sc = score(q, k, d, r, c, scale, beta);
            if (sc > mx) mx = sc;
        }
    real m = mx, l = 0;
    if (variant == V_SOFTMAX1) {
        if (m < 0) m = 0;
        l = exp(-m);
    }
    for (int c = 0; c < n; ++c)
        if (valid(r, c, n, mask, L)) l += exp(score(q, k, d, r, c, scale, beta) - m);
    *m_out = m;
    *l_out = l;
}

/* Attention weight p[r, c] for a valid element; mr, lr from row_stats. */
static real weight(int variant, real sc, real mr, real lr) {
    if (variant == V_SIGMOID) return sigmoid(sc);
    return exp(sc - mr) / lr;
}

/*
 * dS for one valid element, given p = p[r, c], dp = <dO_r, v_c> and, for
 * the softmax family, Dr = sum_c' p[r, c'] dp[r, c'].
 * SIGMOID: the Jacobian of an element-wise sigmoid is diagonal with entries
 * sigma (1 - sigma) (single-cell page, section 2.B).
 * SOFTMAX / SOFTMAX1: dS = p (dp - Dr); both share the Jacobian
 * diag(p) - p p^T, which follows from their definitions.
 */
static real dscore(int variant, real p, real dp, real Dr) {
    if (variant == V_SIGMOID) return dp * p * ((real)1 - p);
    return p * (dp - Dr);
}

static real row_D(int L, int d, int n, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const uint16_t *dout, const uint8_t *mask, int variant, real scale, real beta,
                  int r, real mr, real lr) {
    real D = 0;
    for (int c = 0; c < n; ++c) {
        if (!valid(r, c, n, mask, L)) continue;
        real p = weight(variant, score(q, k, d, r, c, scale, beta), mr, lr);
        D += p * dot_bf16(dout + (size_t)r * d, v + (size_t)c * d, d);
    }
    return D;
}

/*
 * D of one softmax-family row: rowsum(dO_r * o_r).  With the exact output
 * (o == NULL) it is sum_c p[r, c] dp[r, c] (row_D); when the backward is
 * handed a stored output o (bf16 bits [L, d], as the library's backward takes
 * the forward's bf16 O), D is formed from that o, which is what the backward
 * computes with.
 */
static real row_D_given(int L, int d, int n, const uint16_t *q, const uint16_t *k,
                        const uint16_t *v, const uint16_t *dout, const uint16_t *o,
                        const uint8_t *mask, int variant, real scale, real beta, int r, real mr,
                        real lr) {
    if (o == NULL) return row_D(L, d, n, q, k, v, dout, mask, variant, scale, beta, r, mr, lr);
    return dot_bf16(dout + (size_t)r * d, o + (size_t)r * d, d);
}

/*
 * Backward, query side: dQ rows [r0, r1) of one head.
 *   dQ_r = scale * sum_c dS[r, c] k_c;  0 for padded rows.
 * dout: [L, d] bf16 bits; o: the output the backward is given (bf16 bits
 * [L, d]) or NULL for the exact one (softmax family only).  dq: [(r1 - r0), d].
 */
void FN(oracle_bwd_dq_rows)(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const uint16_t *dout, const uint16_t *o,
                            const uint8_t *mask, int bias_mode, int variant, real scale, int r0,
                            int r1, real *dq) {
    int n = clamp_len(seq_len, L);
    real beta = n > 0 ? bias_value(bias_mode, n, L) : (real)0;
    for (int r = r0; r < r1; ++r) {
        real *g = dq + (size_t)(r - r0) * d;
        for (int t = 0; t < d; ++t) g[t] = 0;
        if (r >= n) continue;
        real mr = 0, lr = 1, Dr = 0;
        if (variant != V_SIGMOID) {
            row_stats(L, d, n, q, k, mask, variant, scale, beta, r, &mr, &lr);
            if (lr == 0) continue; /* softmax row with no valid key */
            Dr = row_D_given(L, d, n, q, k, v, dout, o, mask, variant, scale, beta, r, mr, lr);
        }
        for (int c = 0; c < n; ++c) {
            if (!valid(r, c, n, mask, L)) continue;
            real p = weight(variant, score(q, k, d, r, c, scale, beta), mr, lr);
            real dp = dot_bf16(dout + (size_t)r * d, v + (size_t)c * d, d);
            real ds = dscore(variant, p, dp, Dr);
            for (int t = 0; t < d; ++t) g[t] += scale * ds * widen(k[(size_t)c * d + t]);
        }
    }
}

/*
 * Backward, key side: dK and dV rows [c0, c1) of one head.
 *   dV_c = sum_r p[r, c] dO_r;  dK_c = scale * sum_r dS[r, c] q_r;
 * 0 for padded key rows.  The bias is a constant and gets no gradient.
 */
void FN(oracle_bwd_dkv_rows)(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, const uint16_t *dout, const uint16_t *o,
                             const uint8_t *mask, int bias_mode, int variant, real scale, int c0,
                             int c1, real *dk, real *dv) {
    int n = clamp_len(seq_len, L);
    real beta = n > 0 ? bias_value(bias_mode, n, L) : (real)0;
    real *mr = (real *)calloc((size_t)(n > 0 ? n : 1), sizeof(real));
    real *lr = (real *)calloc((size_t)(n > 0 ? n : 1), sizeof(real));
    real *Dr = (real *)calloc((size_t)(n > 0 ? n : 1), sizeof(real));
    if (variant != V_SIGMOID)
        for (int r = 0; r < n; ++r) {
            row_stats(L, d, n, q, k, mask, variant, scale, beta, r, &mr[r], &lr[r]);
            if (lr[r] != 0)
                Dr[r] = row_D_given(L, d, n, q, k, v, dout, o, mask, variant, scale, beta, r,
                                    mr[r], lr[r]);
        }
    for (int c = c0; c < c1; ++c) {
        real *gk = dk + (size_t)(c - c0) * d;
        real *gv = dv + (size_t)(c - c0) * d;
        for (int t = 0; t < d; ++t) gk[t] = gv[t] = 0;
        if (c >= n) continue;
        for (int r = 0; r < n; ++r) {
            if (!valid(r, c, n, mask, L)) continue;
            real p = weight(variant, score(q, k, d, r, c, scale, beta), mr[r], lr[r]);
            real dp = dot_bf16(dout + (size_t)r * d, v + (size_t)c * d, d);
            real ds = dscore(variant, p, dp, Dr[r]);
            for (int t = 0; t < d; ++t) {
                gv[t] += p * widen(dout[(size_t)r * d + t]);
                gk[t] += scale * ds * widen(q[(size_t)r * d + t]);
            }
        }
    }
    free(Dr);
    free(lr);
    free(mr);
}
