/*
 * TEST INFRASTRUCTURE ONLY.  Calls every oracle entry point on small inputs
 * (lengths L, short, 1, 0 and past L; element masks with empty rows; every
 * variant and bias mode; block sizes that clip the last tile) so that a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer can check the oracle's
 * own memory accesses and arithmetic.  Prints "ok" and exits 0 when nothing
 * was reported.  Built and run by tests/test_oracle_sanitizers.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_blockmask(const int32_t *seq_lens, const uint8_t *mask, int B, int L, int bq, int bk,
                      uint8_t *out);
void oracle_fwd_rows_f64(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const uint8_t *mask, int bias_mode, int variant,
                         double scale, int r0, int r1, double *o, double *lse);
void oracle_fwd_tiled_f64(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                          const uint16_t *v, const uint8_t *mask, const uint8_t *bm, int bq,
                          int bk, int bias_mode, int variant, double scale, double *o,
                          double *lse);
void oracle_bwd_dq_rows_f64(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, const uint16_t *dout, const uint16_t *o,
                            const uint8_t *mask, int bias_mode, int variant, double scale, int r0,
                            int r1, double *dq);
void oracle_bwd_dkv_rows_f64(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, const uint16_t *dout, const uint16_t *o,
                             const uint8_t *mask, int bias_mode, int variant, double scale,
                             int c0, int c1, double *dk, double *dv);
void oracle_fwd_rows_f32(int L, int d, int seq_len, const uint16_t *q, const uint16_t *k,
                         const uint16_t *v, const uint8_t *mask, int bias_mode, int variant,
                         float scale, int r0, int r1, float *o, float *lse);

static uint32_t state = 12345u;
static uint16_t rand_bf16(void) {  /* bf16 bits of a value in [-2, 2) */
    state = state * 1664525u + 1013904223u;
    float x = ((float)(state >> 8) / 16777216.0f) * 4.0f - 2.0f;
    union { float f; uint32_t u; } c = {x};
    return (uint16_t)(c.u >> 16);
}

int main(void) {
    const int L = 45, d = 8, B = 4;
    const int32_t lens[4] = {L, 17, 1, 0};
    const int32_t odd[3] = {-3, L + 9, 31};
    uint16_t *q = malloc(sizeof(uint16_t) * L * d), *k = malloc(sizeof(uint16_t) * L * d);
    uint16_t *v = malloc(sizeof(uint16_t) * L * d), *dout = malloc(sizeof(uint16_t) * L * d);
    for (int i = 0; i < L * d; ++i) {
        q[i] = rand_bf16(); k[i] = rand_bf16(); v[i] = rand_bf16(); dout[i] = rand_bf16();
    }
    uint8_t *mask = malloc((size_t)B * L * L);
    for (int i = 0; i < B * L * L; ++i) mask[i] = (uint8_t)((rand_bf16() & 3) != 0);
    for (int c = 0; c < L; ++c) mask[5 * L + c] = 0;  /* a row without a key */
    const int blocks[3][2] = {{32, 32}, {64, 32}, {32, 128}};
    double *o = malloc(sizeof(double) * L * d), *lse = malloc(sizeof(double) * L);
    double *g1 = malloc(sizeof(double) * L * d), *g2 = malloc(sizeof(double) * L * d);
    float *of = malloc(sizeof(float) * L * d), *lf = malloc(sizeof(float) * L);
    double sum = 0.0;
    for (int bi = 0; bi < 3; ++bi) {
        const int bq = blocks[bi][0], bk = blocks[bi][1];
        const int Tq = (L + bq - 1) / bq, Tk = (L + bk - 1) / bk;
        uint8_t *bm = malloc((size_t)B * Tq * Tk);
        oracle_blockmask(lens, mask, B, L, bq, bk, bm);
        oracle_blockmask(lens, NULL, B, L, bq, bk, bm);
        oracle_blockmask(lens, mask, B, L, bq, bk, bm);
        for (int b = 0; b < B + 3; ++b) {
            const int n = b < B ? lens[b] : odd[b - B];
            const uint8_t *mb = b < B ? mask + (size_t)b * L * L : NULL;
            for (int variant = 0; variant < 3; ++variant)
                for (int bias = 0; bias < 3; ++bias) {
                    oracle_fwd_rows_f64(L, d, n, q, k, v, mb, bias, variant, 0.35, 0, L, o, lse);
                    oracle_fwd_tiled_f64(L, d, n, q, k, v, mb, b < B ? bm + (size_t)b * Tq * Tk : NULL,
                                         bq, bk, bias, variant, 0.35, o, lse);
                    for (int given = 0; given < 2; ++given) {  /* exact O, then a given O */
                        const uint16_t *og = given ? v : NULL;
                        oracle_bwd_dq_rows_f64(L, d, n, q, k, v, dout, og, mb, bias, variant, 0.35,
                                               0, L, g1);
                        oracle_bwd_dkv_rows_f64(L, d, n, q, k, v, dout, og, mb, bias, variant,
                                                0.35, 0, L, g1, g2);
                    }
                    oracle_fwd_rows_f32(L, d, n, q, k, v, mb, bias, variant, 0.35f, 3, 9, of, lf);
                    for (int i = 0; i < L * d; ++i) sum += isfinite(g1[i]) ? g1[i] : 0.0;
                }
        }
        free(bm);
    }
    printf("ok %.3f\n", sum);
    free(q); free(k); free(v); free(dout); free(mask); free(o); free(lse); free(g1); free(g2);
    free(of); free(lf);
    return 0;
}
