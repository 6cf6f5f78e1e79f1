/*
 * gdn_oracle.c -- plain, slow fp64 reference of the Gated DeltaNet prefill
 * path (pre -> scan -> post).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the HIP kernels are
 * compared against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header or constant with the GPU
 * library and includes nothing from it.
 *
 * Every quantity is double precision.  Every sum runs in plain index order.
 * Each output element is written by exactly one OpenMP thread, so a result
 * does not depend on the thread count.
 *
 * Sources.  The pages are optimisation audits of an Apple-Metal GDN prompt
 * path.  They name the stages and buffers but print no formula:
 *   - "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1:
 *     gdn_pre runs a 4-tap conv loop with separate paths for the first three
 *     tokens (taps reach into the carried history) and writes the history at
 *     the last token.  It then forms the per-key-head sums of squares of q and
 *     k.  gdn_scan keeps a per-value-head state and updates it in the same loop
 *     that accumulates the two dot products against the old state.  gdn_post
 *     reduces one sum of squares per (token, value head) and applies gamma and
 *     a sigmoid gate.
 *   - "round 10 track b: gdn vectorization and scan", "source and execution":
 *     production width hk=16, hv=48, 10240 channels, eps=1e-6.
 *   - same page, "variants": the conv has exactly four ordered multiply-adds
 *     per element, SiLU also applies to the value channels, and the history
 *     is written back as whole channel rows by the last token.
 * The arithmetic below is the standard Gated DeltaNet layer written out as
 * plainly as possible.  Where the pages leave a step open, the reading taken
 * is noted at that step.
 *
 * Layouts (row-major, C order):
 *   qkv     [T_total][C],  C = 2*hk*dk + hv*dv, channel blocks q | k | v,
 *           head i of a block at [i*d, (i+1)*d)
 *   conv_w  [C][4]         tap m multiplies row (t - 3 + m); tap 3 is the
 *                          current token
 *   hist    [n_seq][3][C]  oldest row first
 *   qn, kn  [T_total][hk][dk]
 *   vc, o   [T_total][hv][dv]
 *   g, beta [T_total][hv]
 *   S       [n_seq][hv][dv][dk]   row index = value index i, column = key j
 *   y, z    [T_total][hv][dv]
 *   cu      [n_seq + 1]    sequence n owns tokens [cu[n], cu[n+1])
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ */
/* Thread control (for timing the oracle on a stated number of cores). */

void gdn_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ */
/* Scalar functions, each taken from its textbook definition.          */

/* logistic sigmoid 1 / (1 + e^-x) */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* SiLU(x) = x * sigmoid(x) */
static double silu(double x) { return x * sigmoid(x); }

/* softplus(x) = ln(1 + e^x), written in the overflow-free form
 * max(x, 0) + ln(1 + e^-|x|). */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

/* ------------------------------------------------------------------ */
/* Step 1: causal depthwise conv with carried history.
 *
 * Round 30 Track C Audit, section 1 (gdn_pre): a 4-tap loop over each channel.
 * The first three tokens of a call take some taps from the carried history.
 * round 10 track b, "variants": four ordered multiply-adds per element.
 *
 * Per sequence n with T_n tokens, the extended input is
 *   Xbar = [hist[n] (3 rows); qkv rows of n (T_n rows)],
 * and for local token tau and channel c
 *   out[tau][c] = sum_{m=0..3} w[c][m] * Xbar[tau + m][c],
 * summed in m order.
 * Reading taken: the pages do not fix the tap orientation.  This is the
 * causal cross-correlation convention: w[c][3] multiplies the current token
 * and w[c][0] the token three steps back.  There is no bias. */
void gdn_oracle_conv(int C, int n_seq, const int64_t *cu,
                     const double *qkv, const double *conv_w,
                     const double *hist, double *out)
{
    for (int n = 0; n < n_seq; ++n) {
        const int64_t t0 = cu[n], T = cu[n + 1] - cu[n];
#pragma omp parallel for schedule(static)
        for (int64_t tau = 0; tau < T; ++tau) {
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int m = 0; m < 4; ++m) {
                    const int64_t r = tau + m; /* row of Xbar */
                    const double x = (r < 3)
                        ? hist[((size_t)n * 3 + (size_t)r) * C + c]
                        : qkv[(size_t)(t0 + r - 3) * C + c];
                    acc += conv_w[(size_t)c * 4 + m] * x;
                }
                out[(size_t)(t0 + tau) * C + c] = acc;
            }
        }
    }
}

/* Step 1b: the carried history after the call is the last three rows of
 * Xbar, i.e. Xbar[T_n .. T_n + 2].
 * Round 30 Track C Audit, section 1: the last token writes the history.
 * Reading taken: when T_n < 3 the newest rows come from this call and the
 * older ones are history rows kept from before; T_n = 0 leaves it unchanged. */
void gdn_oracle_history(int C, int n_seq, const int64_t *cu,
                        const double *qkv, const double *hist_in,
                        double *hist_out)
{
    for (int n = 0; n < n_seq; ++n) {
        const int64_t t0 = cu[n], T = cu[n + 1] - cu[n];
        for (int r = 0; r < 3; ++r) {
            const int64_t src = T + r; /* row of Xbar */
            for (int c = 0; c < C; ++c) {
                hist_out[((size_t)n * 3 + r) * C + c] = (src < 3)
                    ? hist_in[((size_t)n * 3 + (size_t)src) * C + c]
                    : qkv[(size_t)(t0 + src - 3) * C + c];
            }
        }
    }
}

/* Step 2: SiLU on every conv output.  round 10 track b, "variants": SiLU
 * also applies to the value channels. */
void gdn_oracle_silu(int64_t n, const double *x, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = silu(x[i]);
}

/* Step 3: L2 normalisation of one head vector of length d:
 *   y = x / sqrt(sum_i x_i^2 + eps).
 * Round 30 Track C Audit, section 1: one sum of squares per key head for q
 * and one for k.  Reading taken: eps sits inside the square root, added to
 * the sum of squares. */
void gdn_oracle_l2norm(int64_t n_vec, int d, const double *x, double eps,
                       double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t v = 0; v < n_vec; ++v) {
        const double *xv = x + (size_t)v * d;
        double ss = 0.0;
        for (int i = 0; i < d; ++i) ss += xv[i] * xv[i];
        const double inv = 1.0 / sqrt(ss + eps);
        for (int i = 0; i < d; ++i) y[(size_t)v * d + i] = xv[i] * inv;
    }
}

/* Step 4: gates, per token t and value head h:
 *   g    = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h])   (log decay)
 *   beta = sigmoid(b[t][h])
 * The pages keep both in one per-value-head buffer (gb, stride hv). */
void gdn_oracle_gates(int64_t T, int hv, const double *a, const double *b,
                      const double *A_log, const double *dt_bias,
                      double *g, double *beta)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int h = 0; h < hv; ++h) {
            const size_t i = (size_t)t * hv + h;
            g[i] = -exp(A_log[h]) * softplus(a[i] + dt_bias[h]);
            beta[i] = sigmoid(b[i]);
        }
    }
}

/* The whole pre stage: conv -> SiLU -> split into q | k | v -> L2 norm of q
 * and k per key head -> gates; plus the history carry.  `work` must hold
 * 2 * T_total * C doubles. */
void gdn_oracle_pre(int hk, int hv, int dk, int dv, int n_seq,
                    const int64_t *cu, const double *qkv,
                    const double *conv_w, const double *a, const double *b,
                    const double *A_log, const double *dt_bias,
                    const double *hist_in, double eps_l2, double *qn,
                    double *kn, double *vc, double *g, double *beta,
                    double *hist_out, double *work)
{
    const int C = 2 * hk * dk + hv * dv;
    const int64_t T = cu[n_seq];
    double *xc = work;                 /* conv output */
    double *xs = work + (size_t)T * C; /* after SiLU */
    gdn_oracle_conv(C, n_seq, cu, qkv, conv_w, hist_in, xc);
    gdn_oracle_silu(T * (int64_t)C, xc, xs);

    /* split: gather each block of channels into its own array */
    for (int64_t t = 0; t < T; ++t) {
        const double *row = xs + (size_t)t * C;
        memcpy(qn + (size_t)t * hk * dk, row, sizeof(double) * hk * dk);
        memcpy(kn + (size_t)t * hk * dk, row + hk * dk,
               sizeof(double) * hk * dk);
        memcpy(vc + (size_t)t * hv * dv, row + 2 * hk * dk,
               sizeof(double) * hv * dv);
    }
    /* normalise q and k in place, one key head at a time */
    gdn_oracle_l2norm(T * hk, dk, qn, eps_l2, qn);
    gdn_oracle_l2norm(T * hk, dk, kn, eps_l2, kn);
    gdn_oracle_gates(T, hv, a, b, A_log, dt_bias, g, beta);
    gdn_oracle_history(C, n_seq, cu, qkv, hist_in, hist_out);
}

/* ------------------------------------------------------------------ */
/* Step 5: the gated delta rule, per sequence and value head.
 *
 * Round 30 Track C Audit, section 1 (gdn_scan_r findings): one fp32 state
 * per value head, updated token by token in the same loop that forms the
 * two dot products against the old state.  The arithmetic, for value head h
 * reading key head j = h / (hv / hk) and a dv x dk state S:
 *   alpha_t = exp(g_t)
 *   A       = alpha_t * S_{t-1}                 (decay)
 *   p       = A k_t                             (what the state predicts)
 *   u       = beta_t * (v_t - p)                (delta-rule correction)
 *   S_t     = A + u k_t^T                       (rank-1 write)
 *   o_t     = S_t q_t / sqrt(dk)
 * Reading taken: value heads map to key heads in contiguous groups (h / G,
 * not h mod hk), and 1/sqrt(dk) scales the output.
 *
 * S_in and S_out may be the same buffer.  If `heads` is non-NULL, only the
 * n_heads listed value heads are run (for sampled checks of large
 * workloads); o and S_out of the other heads are left untouched. */
void gdn_oracle_scan(int hk, int hv, int dk, int dv, int n_seq,
                     const int64_t *cu, const double *qn, const double *kn,
                     const double *vc, const double *g, const double *beta,
                     const double *S_in, double *S_out, double *o,
                     const int32_t *heads, int n_heads)
{
    const int G = hv / hk;
    const int nh = heads ? n_heads : hv;
    const double scale = 1.0 / sqrt((double)dk);
    const size_t SS = (size_t)dv * dk;

#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int n = 0; n < n_seq; ++n) {
        for (int hi = 0; hi < nh; ++hi) {
            const int h = heads ? heads[hi] : hi;
            const int j = h / G;
            double *S = (double *)malloc(sizeof(double) * SS);
            double *u = (double *)malloc(sizeof(double) * dv);
            memcpy(S, S_in + ((size_t)n * hv + h) * SS, sizeof(double) * SS);
            for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
                const double alpha = exp(g[(size_t)t * hv + h]);
                const double bt = beta[(size_t)t * hv + h];
                const double *k = kn + ((size_t)t * hk + j) * dk;
                const double *q = qn + ((size_t)t * hk + j) * dk;
                const double *v = vc + ((size_t)t * hv + h) * dv;
                for (size_t e = 0; e < SS; ++e) S[e] *= alpha;
                for (int i = 0; i < dv; ++i) {
                    double p = 0.0;
                    for (int c = 0; c < dk; ++c) p += S[(size_t)i * dk + c] * k[c];
                    u[i] = bt * (v[i] - p);
                }
                for (int i = 0; i < dv; ++i)
                    for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += u[i] * k[c];
                double *ot = o + ((size_t)t * hv + h) * dv;
                for (int i = 0; i < dv; ++i) {
                    double acc = 0.0;
                    for (int c = 0; c < dk; ++c) acc += S[(size_t)i * dk + c] * q[c];
                    ot[i] = acc * scale;
                }
            }
            memcpy(S_out + ((size_t)n * hv + h) * SS, S, sizeof(double) * SS);
            free(u);
            free(S);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Step 6: per-head RMSNorm with gamma, times the SiLU output gate.
 *
 * Round 30 Track C Audit, section 1 (gdn_post): one sum of squares per
 * (token, value head) row of dv values.  round 25 track A, "shipped": a
 * sigmoid gate and a gamma load.  For one row o of length dv:
 *   ms  = (1/dv) * sum_i o_i^2
 *   y_i = (o_i / sqrt(ms + eps)) * gamma_i * (z_i * sigmoid(z_i))
 * Readings taken: gamma has dv entries shared by all value heads, eps sits
 * inside the square root, and the order is normalise, then gamma, then
 * gate.  The result is not rounded here; rounding to the output type is the
 * caller's. */
void gdn_oracle_post(int64_t n_rows, int dv, const double *o, const double *z,
                     const double *gamma, double eps, double *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        const double *orow = o + (size_t)r * dv;
        const double *zrow = z + (size_t)r * dv;
        double ss = 0.0;
        for (int i = 0; i < dv; ++i) ss += orow[i] * orow[i];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        for (int i = 0; i < dv; ++i)
            y[(size_t)r * dv + i] = ((orow[i] * inv) * gamma[i]) * silu(zrow[i]);
    }
}
