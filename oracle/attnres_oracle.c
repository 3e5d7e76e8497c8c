/*
 * attnres_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of the Attention Residuals (AttnRes) depth
 * aggregation, used to check the GPU library.  Nothing in the product path may
 * call it; only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no source with the HIP library.
 *
 * Sources (the pages, cited by title and section):
 *   [DB]  "DepthBench: 残差连接如何把网络层数转化为有效计算深度" (reading notes on
 *         arXiv 2609.32534), sec. 2.3 "Full AttnRes" (the e/a/z/f equations and
 *         the paragraph after them), sec. 2.5 "Block AttnRes 与 mHC 的设计取舍".
 *   [LR]  "LLM跨层信息传递优化：DeepSeek mHC & Kimi AttnRes解析", section
 *         "Kimi AttnRes" (the alpha/phi/q/k/v equations, the Block paragraph).
 *   [K3N] "Kimi K3 notes 2: attention residuals" (jaimeyzzz.com), sec. 5
 *         "Attention Residuals：动态选择历史层" (the two-step score/softmax).
 *   [DC]  DataCamp "Attention Residuals explained", sections "块式注意力残差"
 *         (block representation, b_0 = h_1) and the "两阶段计算" system bullet.
 *
 * What is computed, for one token and one read (query) l:
 *   sources X_l                  (Full: v_0..v_l; Block: see block_sources)
 *   r(x)  = 1 / sqrt(mean_k x_k^2 + eps)      RMSNorm of the key, unit gain
 *   s(x)  = r(x) * (w_l . x)                  no 1/sqrt(d), temperature 1 [DB 2.3]
 *   alpha = softmax over X_l of s             [DB 2.3], [K3N 5]
 *   h_l   = sum_x alpha(x) * x                raw values, not normalised [LR]
 *   lse_l = max s + log sum exp(s - max s)
 *
 * Indexing reading (the pages number reads from 1 and let read l see i < l):
 * here read l (0-based) sees history rows 0..l, so read 0 is "the first
 * sublayer reads the embedding directly" and the last read is the LM head's
 * own read [DB 2.3].
 *
 * Block reading: the history is v_0 (embedding) followed by sublayer outputs
 * v_1..; consecutive runs of S sublayer outputs form a block whose summary is
 * their plain sum ([LR] "将内部所有层的输出加和", [DB 2.5] "相加").  Read l with
 * m = floor(l/S) sees [v_0, b_1..b_m] plus the running partial sum
 * p_l = v_{mS+1} + ... + v_l when that sum is non-empty ([DC] block section:
 * embedding, earlier block summaries, current partial sum).
 *
 * The backward is not on the pages; it is the derivative of the definition
 * above, written out (derivation in the header of attnres_oracle_bwd below) and
 * pinned by finite differences in the tests.
 *
 * Inputs are double arrays (the callers upcast bf16 / fp32 values exactly);
 * every arithmetic step is in double.  Parallel over tokens with OpenMP; the
 * per-token arithmetic is strictly sequential in the order written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int attnres_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n >= 1); for timing on one core. */
void attnres_oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Block membership of read l: number of completed blocks m and the half-open
 * row range [part_begin, part_end) of the partial sum (empty when equal). */
void attnres_oracle_block_sources(int64_t l, int64_t S, int64_t* m_out,
                                  int64_t* part_begin, int64_t* part_end) {
    int64_t m = l / S;
    *m_out = m;
    *part_begin = m * S + 1;
    *part_end = l + 1;
}

/* Number of sources read l sees. */
int64_t attnres_oracle_num_sources(int variant, int64_t l, int64_t S) {
    if (variant == 0) return l + 1;
    int64_t m, pb, pe;
    attnres_oracle_block_sources(l, S, &m, &pb, &pe);
    return 1 + m + (pe > pb ? 1 : 0);
}

/* Build the source vectors of read l for token t into src[n_src][d].
 * hist is [n_hist][T][d].  Also records, for each source, the half-open range
 * of history rows it sums (rows_lo/rows_hi), so the backward can route the
 * gradient of a source to every row inside it. */
static int64_t build_sources(int variant, int64_t S, const double* hist, int64_t T,
                             int64_t d, int64_t l, int64_t t, double* src,
                             int64_t* rows_lo, int64_t* rows_hi) {
    int64_t n = 0;
    if (variant == 0) {
        for (int64_t i = 0; i <= l; ++i) {
            const double* v = hist + (i * T + t) * d;
            for (int64_t k = 0; k < d; ++k) src[n * d + k] = v[k];
            rows_lo[n] = i;
            rows_hi[n] = i + 1;
            ++n;
        }
        return n;
    }
    int64_t m, pb, pe;
    attnres_oracle_block_sources(l, S, &m, &pb, &pe);
    /* v_0: the embedding is a source of its own (b_0 = h_1 in [DC]). */
    {
        const double* v = hist + (0 * T + t) * d;
        for (int64_t k = 0; k < d; ++k) src[k] = v[k];
        rows_lo[0] = 0;
        rows_hi[0] = 1;
        n = 1;
    }
    /* completed blocks b_1..b_m: plain sums of S consecutive sublayer outputs */
    for (int64_t c = 1; c <= m; ++c) {
        double* b = src + n * d;
        for (int64_t k = 0; k < d; ++k) b[k] = 0.0;
        for (int64_t i = (c - 1) * S + 1; i <= c * S; ++i) {
            const double* v = hist + (i * T + t) * d;
            for (int64_t k = 0; k < d; ++k) b[k] += v[k];
        }
        rows_lo[n] = (c - 1) * S + 1;
        rows_hi[n] = c * S + 1;
        ++n;
    }
    /* the running partial sum of the current block, if non-empty */
    if (pe > pb) {
        double* p = src + n * d;
        for (int64_t k = 0; k < d; ++k) p[k] = 0.0;
        for (int64_t i = pb; i < pe; ++i) {
            const double* v = hist + (i * T + t) * d;
            for (int64_t k = 0; k < d; ++k) p[k] += v[k];
        }
        rows_lo[n] = pb;
        rows_hi[n] = pe;
        ++n;
    }
    return n;
}

/* r(x) = 1/sqrt(mean(x^2) + eps): the RMSNorm scale of a key, unit gain. */
static double rms_inv(const double* x, int64_t d, double eps) {
    double ss = 0.0;
    for (int64_t k = 0; k < d; ++k) ss += x[k] * x[k];
    return 1.0 / sqrt(ss / (double)d + eps);
}

static double dot(const double* a, const double* b, int64_t d) {
    double s = 0.0;
    for (int64_t k = 0; k < d; ++k) s += a[k] * b[k];
    return s;
}

/* Pre-norm of each read's mixture: the sublayer's branch input
 * RMSNorm_pre,l(z_l) ([DB] sec. 2.3, the f_l equation), with the same RMSNorm
 * as the keys (r = 1/sqrt(mean z^2 + eps)) and a per-read gain vector:
 *   y[l][t] = gain[l] * z[l][t] * r(z[l][t])      (gain NULL: unit gain)
 *   z, y [n_q][T][d];  gain [n_q][d] or NULL.  Returns 0, or -1 on bad sizes. */
int attnres_oracle_prenorm(const double* z, int64_t n_q, int64_t T, int64_t d,
                           const double* gain, double eps, double* y) {
    if (n_q < 0 || T < 0 || d < 1 || !(eps >= 0.0)) return -1;
    for (int64_t j = 0; j < n_q; ++j) {
        for (int64_t t = 0; t < T; ++t) {
            const double* zr = z + (j * T + t) * d;
            double* yr = y + (j * T + t) * d;
            const double r = rms_inv(zr, d, eps);
            for (int64_t k = 0; k < d; ++k) yr[k] = (gain ? gain[j * d + k] : 1.0) * zr[k] * r;
        }
    }
    return 0;
}

/* Single-pass forward for Full (variant 0) or Block (variant 1).
 *   hist  [n_hist][T][d]   w [n_q][d] (row j is read q_begin + j)
 *   out   [n_q][T][d]      lse [n_q][T] or NULL
 *   alpha [n_q][T][n_hist] or NULL: softmax weights, in source order,
 *         zero-padded past the read's source count.
 * Returns 0, or -1 on bad arguments / allocation failure. */
static int fwd_impl(int variant, int64_t S, const double* hist, int64_t n_hist,
                    int64_t T, int64_t d, const double* w, int per_token, int64_t q_begin,
                    int64_t n_q, double eps, double* out, double* lse, double* alpha);

int attnres_oracle_fwd(int variant, int64_t S, const double* hist, int64_t n_hist,
                       int64_t T, int64_t d, const double* w, int64_t q_begin,
                       int64_t n_q, double eps, double* out, double* lse,
                       double* alpha) {
    return fwd_impl(variant, S, hist, n_hist, T, d, w, 0, q_begin, n_q, eps, out, lse, alpha);
}

/* The same forward with an input-dependent query per (read, token)
 * ("Kimi K3 notes 2" sec. 6, the ablation): q [n_q][T][d], row (j, t) is the
 * query of read q_begin + j for token t. */
int attnres_oracle_fwd_tokq(int variant, int64_t S, const double* hist, int64_t n_hist,
                            int64_t T, int64_t d, const double* q, int64_t q_begin,
                            int64_t n_q, double eps, double* out, double* lse) {
    return fwd_impl(variant, S, hist, n_hist, T, d, q, 1, q_begin, n_q, eps, out, lse, NULL);
}

/* Input-dependent query projection: q[j][t] = W[j] x[j][t], with
 * W [n_q][d][d] row-major (q_k = sum_i W[j][k][i] x_i) and x [n_q][T][d] the
 * hidden state each read projects from. */
int attnres_oracle_query_proj(const double* x, const double* W, int64_t n_q, int64_t T,
                              int64_t d, double* q) {
    if (n_q < 0 || T < 0 || d < 1) return -1;
    for (int64_t j = 0; j < n_q; ++j)
        for (int64_t t = 0; t < T; ++t) {
            const double* xr = x + (j * T + t) * d;
            double* qr = q + (j * T + t) * d;
            for (int64_t k = 0; k < d; ++k) {
                const double* wr = W + (j * d + k) * d;
                double s = 0.0;
                for (int64_t i = 0; i < d; ++i) s += wr[i] * xr[i];
                qr[k] = s;
            }
        }
    return 0;
}

static int fwd_impl(int variant, int64_t S, const double* hist, int64_t n_hist,
                    int64_t T, int64_t d, const double* w, int per_token, int64_t q_begin,
                    int64_t n_q, double eps, double* out, double* lse, double* alpha) {
    if (variant != 0 && variant != 1) return -1;
    if (variant == 1 && S < 1) return -1;
    if (n_hist < 1 || T < 0 || d < 1 || q_begin < 0 || n_q < 0 ||
        q_begin + n_q > n_hist)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double* src = (double*)malloc(sizeof(double) * (size_t)(n_hist * d));
        double* s = (double*)malloc(sizeof(double) * (size_t)n_hist);
        int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_hist);
        int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_hist);
        int ok = 1;
        if (!src || !s || !lo || !hi) {
            ok = 0;
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!ok) continue;
            for (int64_t j = 0; j < n_q; ++j) {
                int64_t l = q_begin + j;
                const double* wl = per_token ? w + (j * T + t) * d : w + j * d;
                int64_t n = build_sources(variant, S, hist, T, d, l, t, src, lo, hi);
                /* scores s(x) = r(x) * (w_l . x) */
                double smax = -INFINITY;
                for (int64_t x = 0; x < n; ++x) {
                    const double* xv = src + x * d;
                    double r = rms_inv(xv, d, eps);
                    double wx = 0.0;
                    for (int64_t k = 0; k < d; ++k) wx += wl[k] * xv[k];
                    s[x] = r * wx;
                    if (s[x] > smax) smax = s[x];
                }
                /* softmax over depth, max-subtracted */
                double z = 0.0;
                for (int64_t x = 0; x < n; ++x) z += exp(s[x] - smax);
                double* h = out + (j * T + t) * d;
                for (int64_t k = 0; k < d; ++k) h[k] = 0.0;
                for (int64_t x = 0; x < n; ++x) {
                    double a = exp(s[x] - smax) / z;
                    const double* xv = src + x * d;
                    for (int64_t k = 0; k < d; ++k) h[k] += a * xv[k];
                    if (alpha) alpha[(j * T + t) * n_hist + x] = a;
                }
                if (alpha)
                    for (int64_t x = n; x < n_hist; ++x)
                        alpha[(j * T + t) * n_hist + x] = 0.0;
                if (lse) lse[j * T + t] = smax + log(z);
            }
        }
        free(src);
        free(s);
        free(lo);
        free(hi);
    }
    return failed ? -1 : 0;
}

/* Two-phase Block forward ([DC], "两阶段计算"): for the reads of one block
 * group m, phase 1 attends over the frozen sources C_m = [v_0, b_1..b_m] alone
 * and keeps (M1, Z1, o) = (max score, sum exp(s - M1), normalised weighted
 * sum); phase 2 scores the partial sum p_l and merges it by the log-sum-exp
 * rule:
 *   M = max(M1, s_p),  A = Z1 exp(M1 - M),  B = exp(s_p - M)
 *   h = (A o + B p) / (A + B),  lse = M + log(A + B).
 * With an empty partial, h = o and lse = M1 + log Z1.  Same arguments as the
 * single-pass routine with variant = 1 (no alpha output). */
int attnres_oracle_block_fwd_twophase(int64_t S, const double* hist, int64_t n_hist,
                                      int64_t T, int64_t d, const double* w,
                                      int64_t q_begin, int64_t n_q, double eps,
                                      double* out, double* lse) {
    if (S < 1 || n_hist < 1 || T < 0 || d < 1 || q_begin < 0 || n_q < 0 ||
        q_begin + n_q > n_hist)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double* src = (double*)malloc(sizeof(double) * (size_t)(n_hist * d));
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_hist);
        int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_hist);
        int ok = 1;
        if (!src || !o || !lo || !hi) {
            ok = 0;
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!ok) continue;
            for (int64_t j = 0; j < n_q; ++j) {
                int64_t l = q_begin + j;
                const double* wl = w + j * d;
                int64_t n = build_sources(1, S, hist, T, d, l, t, src, lo, hi);
                int64_t m, pb, pe;
                attnres_oracle_block_sources(l, S, &m, &pb, &pe);
                int64_t n1 = 1 + m; /* sources of phase 1 */
                int has_p = (pe > pb);
                /* phase 1 over C_m */
                double M1 = -INFINITY;
                for (int64_t x = 0; x < n1; ++x) {
                    double sx = rms_inv(src + x * d, d, eps) * dot(src + x * d, wl, d);
                    if (sx > M1) M1 = sx;
                }
                double Z1 = 0.0;
                for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
                for (int64_t x = 0; x < n1; ++x) {
                    double sx = rms_inv(src + x * d, d, eps) * dot(src + x * d, wl, d);
                    double e = exp(sx - M1);
                    Z1 += e;
                    for (int64_t k = 0; k < d; ++k) o[k] += e * src[x * d + k];
                }
                for (int64_t k = 0; k < d; ++k) o[k] /= Z1;
                double* h = out + (j * T + t) * d;
                if (!has_p) {
                    for (int64_t k = 0; k < d; ++k) h[k] = o[k];
                    if (lse) lse[j * T + t] = M1 + log(Z1);
                    continue;
                }
                /* phase 2: merge the partial sum p_l */
                const double* p = src + (n - 1) * d;
                double sp = rms_inv(p, d, eps) * dot(p, wl, d);
                double M = M1 > sp ? M1 : sp;
                double A = Z1 * exp(M1 - M);
                double B = exp(sp - M);
                for (int64_t k = 0; k < d; ++k) h[k] = (A * o[k] + B * p[k]) / (A + B);
                if (lse) lse[j * T + t] = M + log(A + B);
            }
        }
        free(src);
        free(o);
        free(lo);
        free(hi);
    }
    return failed ? -1 : 0;
}

/* Backward of the forward above (not stated on the pages; derived here).
 *
 * For one token and read l with upstream gradient g = dL/dh_l:
 *   h = sum_x alpha_x x,  alpha = softmax(s),  s_x = r_x (w . x),
 *   r_x = (|x|^2/d + eps)^(-1/2).
 *   dL/dalpha_x = g . x                                  (=: a_x)
 *   dL/ds_x     = alpha_x (a_x - sum_y alpha_y a_y)       (softmax Jacobian)
 *   ds_x/dx     = r_x w - (r_x^2 s_x / d) x               (since dr/dx = -r^3 x/d)
 *   ds_x/dw     = r_x x
 * so
 *   dL/dx  += alpha_x g + dL/ds_x (r_x w - (r_x^2 s_x/d) x)
 *   dL/dw_l += sum_x dL/ds_x r_x x.
 * A source that is a sum of history rows (a block summary or a partial sum)
 * passes its gradient unchanged to every row in it.
 *
 *   dout  [n_q][T][d]   dhist [n_hist][T][d] (overwritten)   dw [n_q][d] (overwritten)
 */
int attnres_oracle_bwd(int variant, int64_t S, const double* hist, int64_t n_hist,
                       int64_t T, int64_t d, const double* w, int64_t q_begin,
                       int64_t n_q, double eps, const double* dout, double* dhist,
                       double* dw) {
    if (variant != 0 && variant != 1) return -1;
    if (variant == 1 && S < 1) return -1;
    if (n_hist < 1 || T < 0 || d < 1 || q_begin < 0 || n_q < 0 ||
        q_begin + n_q > n_hist)
        return -1;
    memset(dhist, 0, sizeof(double) * (size_t)(n_hist * T * d));
    int nthr = attnres_oracle_num_threads();
    /* per-thread dw partials, summed in thread order at the end */
    double* dw_part = (double*)calloc((size_t)nthr * (size_t)(n_q * d), sizeof(double));
    if (!dw_part) return -1;
    int failed = 0;
#pragma omp parallel
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double* my_dw = dw_part + (size_t)tid * (size_t)(n_q * d);
        double* src = (double*)malloc(sizeof(double) * (size_t)(n_hist * d));
        double* s = (double*)malloc(sizeof(double) * (size_t)n_hist);
        double* r = (double*)malloc(sizeof(double) * (size_t)n_hist);
        double* al = (double*)malloc(sizeof(double) * (size_t)n_hist);
        double* da = (double*)malloc(sizeof(double) * (size_t)n_hist);
        double* dx = (double*)malloc(sizeof(double) * (size_t)d);
        int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_hist);
        int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * (size_t)n_hist);
        int ok = 1;
        if (!src || !s || !r || !al || !da || !dx || !lo || !hi) {
            ok = 0;
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            if (!ok) continue;
            for (int64_t j = 0; j < n_q; ++j) {
                int64_t l = q_begin + j;
                const double* wl = w + j * d;
                const double* g = dout + (j * T + t) * d;
                int64_t n = build_sources(variant, S, hist, T, d, l, t, src, lo, hi);
                double smax = -INFINITY;
                for (int64_t x = 0; x < n; ++x) {
                    r[x] = rms_inv(src + x * d, d, eps);
                    s[x] = r[x] * dot(src + x * d, wl, d);
                    if (s[x] > smax) smax = s[x];
                }
                double z = 0.0;
                for (int64_t x = 0; x < n; ++x) z += exp(s[x] - smax);
                double delta = 0.0;
                for (int64_t x = 0; x < n; ++x) {
                    al[x] = exp(s[x] - smax) / z;
                    da[x] = dot(src + x * d, g, d);
                    delta += al[x] * da[x];
                }
                for (int64_t x = 0; x < n; ++x) {
                    const double* xv = src + x * d;
                    double ds = al[x] * (da[x] - delta);
                    double c = r[x] * r[x] * s[x] / (double)d;
                    for (int64_t k = 0; k < d; ++k)
                        dx[k] = al[x] * g[k] + ds * (r[x] * wl[k] - c * xv[k]);
                    for (int64_t k = 0; k < d; ++k) my_dw[j * d + k] += ds * r[x] * xv[k];
                    /* route to every history row the source sums */
                    for (int64_t i = lo[x]; i < hi[x]; ++i) {
                        double* dv = dhist + (i * T + t) * d;
                        for (int64_t k = 0; k < d; ++k) dv[k] += dx[k];
                    }
                }
            }
        }
        free(src);
        free(s);
        free(r);
        free(al);
        free(da);
        free(dx);
        free(lo);
        free(hi);
    }
    if (!failed) {
        for (int64_t k = 0; k < n_q * d; ++k) {
            double acc = 0.0;
            for (int th = 0; th < nthr; ++th) acc += dw_part[(size_t)th * (size_t)(n_q * d) + k];
            dw[k] = acc;
        }
    }
    free(dw_part);
    return failed ? -1 : 0;
}
