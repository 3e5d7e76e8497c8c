/*
 * Runs every function of the fp64 oracle (oracle/attnres_oracle.c) on small
 * inputs -- Full and Block forwards with the weight probe, the two-phase Block
 * forward, per-token queries, the projection, the pre-norm, the backward, the
 * source indexing -- so that an AddressSanitizer / UndefinedBehaviorSanitizer
 * build checks its memory accesses and arithmetic.  It also checks a few
 * properties that hold for any input (weights sum to one, the two-phase
 * forward equals the single pass, finite gradients).  Test code only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int attnres_oracle_fwd(int variant, int64_t S, const double* hist, int64_t n_hist, int64_t T,
                       int64_t d, const double* w, int64_t q_begin, int64_t n_q, double eps,
                       double* out, double* lse, double* alpha);
int attnres_oracle_fwd_tokq(int variant, int64_t S, const double* hist, int64_t n_hist,
                            int64_t T, int64_t d, const double* q, int64_t q_begin, int64_t n_q,
                            double eps, double* out, double* lse);
int attnres_oracle_block_fwd_twophase(int64_t S, const double* hist, int64_t n_hist, int64_t T,
                                      int64_t d, const double* w, int64_t q_begin, int64_t n_q,
                                      double eps, double* out, double* lse);
int attnres_oracle_query_proj(const double* x, const double* W, int64_t n_q, int64_t T,
                              int64_t d, double* q);
int attnres_oracle_prenorm(const double* z, int64_t n_q, int64_t T, int64_t d,
                           const double* gain, double eps, double* y);
int attnres_oracle_bwd(int variant, int64_t S, const double* hist, int64_t n_hist, int64_t T,
                       int64_t d, const double* w, int64_t q_begin, int64_t n_q, double eps,
                       const double* dout, double* dhist, double* dw);
void attnres_oracle_block_sources(int64_t l, int64_t S, int64_t* m_out, int64_t* part_begin,
                                  int64_t* part_end);
int64_t attnres_oracle_num_sources(int variant, int64_t l, int64_t S);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform_pm1(void) { /* xorshift64*, mapped to [-1, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
static double* fill(size_t n, double scale) {
    double* a = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = scale * uniform_pm1();
    return a;
}
static int failures = 0;
#define EXPECT(c)                                                                 \
    do {                                                                          \
        if (!(c)) {                                                               \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c);      \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

int main(void) {
    const int64_t n_hist = 11, T = 5, d = 24;
    double* hist = fill((size_t)(n_hist * T * d), 1.0);
    double* w = fill((size_t)(n_hist * d), 0.4);
    double* dout = fill((size_t)(n_hist * T * d), 1.0);
    double* out = calloc((size_t)(n_hist * T * d), sizeof(double));
    double* out2 = calloc((size_t)(n_hist * T * d), sizeof(double));
    double* lse = calloc((size_t)(n_hist * T), sizeof(double));
    double* lse2 = calloc((size_t)(n_hist * T), sizeof(double));
    double* alpha = calloc((size_t)(n_hist * T * n_hist), sizeof(double));
    for (int variant = 0; variant <= 1; ++variant) {
        for (int64_t S = 1; S <= 12; S += 3) {
            EXPECT(attnres_oracle_fwd(variant, S, hist, n_hist, T, d, w, 0, n_hist, 1e-6, out, lse,
                                      alpha) == 0);
            for (int64_t j = 0; j < n_hist; ++j)
                for (int64_t t = 0; t < T; ++t) {
                    double s = 0.0;
                    for (int64_t x = 0; x < n_hist; ++x) s += alpha[(j * T + t) * n_hist + x];
                    EXPECT(fabs(s - 1.0) < 1e-12);
                }
            /* a read subset */
            EXPECT(attnres_oracle_fwd(variant, S, hist, n_hist, T, d, w + 3 * d, 3, 5, 1e-6, out2,
                                      lse2, NULL) == 0);
            EXPECT(attnres_oracle_fwd_tokq(variant, S, hist, n_hist, T, d, dout, 0, n_hist, 1e-6,
                                           out2, lse2) == 0);
            double* dh = calloc((size_t)(n_hist * T * d), sizeof(double));
            double* dw = calloc((size_t)(n_hist * d), sizeof(double));
            EXPECT(attnres_oracle_bwd(variant, S, hist, n_hist, T, d, w, 0, n_hist, 1e-6, dout, dh,
                                      dw) == 0);
            for (int64_t i = 0; i < n_hist * T * d; ++i) EXPECT(isfinite(dh[i]));
            EXPECT(attnres_oracle_bwd(variant, S, hist, n_hist, T, d, w + 2 * d, 2, 4, 1e-6, dout, dh,
                                      dw) == 0);
            free(dh);
            free(dw);
        }
    }
    for (int64_t S = 1; S <= 12; S += 2) { /* two-phase equals the single pass */
        EXPECT(attnres_oracle_block_fwd_twophase(S, hist, n_hist, T, d, w, 0, n_hist, 1e-6, out2,
                                                 lse2) == 0);
        EXPECT(attnres_oracle_fwd(1, S, hist, n_hist, T, d, w, 0, n_hist, 1e-6, out, lse, NULL) == 0);
        for (int64_t i = 0; i < n_hist * T * d; ++i) EXPECT(fabs(out[i] - out2[i]) < 1e-12);
    }
    double* W = fill((size_t)(3 * d * d), 0.2);
    double* q = calloc((size_t)(3 * T * d), sizeof(double));
    EXPECT(attnres_oracle_query_proj(hist, W, 3, T, d, q) == 0);
    double* gain = fill((size_t)(3 * d), 1.0);
    EXPECT(attnres_oracle_prenorm(out, 3, T, d, gain, 1e-6, out2) == 0);
    EXPECT(attnres_oracle_prenorm(out, 3, T, d, NULL, 1e-6, out2) == 0);
    for (int64_t l = 0; l < 70; ++l)
        for (int64_t S = 1; S < 10; ++S) {
            int64_t m, pb, pe;
            attnres_oracle_block_sources(l, S, &m, &pb, &pe);
            EXPECT(m == l / S && pb == m * S + 1 && pe == l + 1);
            EXPECT(attnres_oracle_num_sources(1, l, S) == m + 1 + (l % S != 0));
        }
    /* rejected arguments */
    EXPECT(attnres_oracle_fwd(0, 1, hist, n_hist, T, d, w, 5, n_hist, 1e-6, out, lse, NULL) != 0);
    EXPECT(attnres_oracle_fwd(1, 0, hist, n_hist, T, d, w, 0, n_hist, 1e-6, out, lse, NULL) != 0);
    free(hist); free(w); free(dout); free(out); free(out2); free(lse); free(lse2); free(alpha);
    free(W); free(q); free(gain);
    printf("oracle driver: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
