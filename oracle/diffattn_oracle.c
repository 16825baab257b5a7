/*
 * Differential attention forward -- CPU oracle in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * this file's library.  It shares no code with the HIP path.
 *
 * Pages cited (all statements below restate them in our own words):
 *   [U]  Ultralytics glossary entry "Differential Transformer" (Japanese, Portuguese and Arabic editions carry the
 *        same text), section on how differential attention works: the worked PyTorch example and the paragraph
 *        after it.
 *   [J]  jisaku.com glossary entry "Differential Transformer (Diff Attention)", section "main features /
 *        mechanism".
 *
 * What one query row computes (plain definition, no blocking, no streaming):
 *   1. Visible keys J: all keys, or with the causal flag the keys j <= i + (Nk - Nq) (query rows aligned to the
 *      end of the key sequence, so a square prefill masks j <= i and a single decode query sees every key).
 *      The pages do not discuss masking; the causal flag follows the lower-triangular reading.
 *   2. Two score vectors s1_j = (q1 . k1_j) / sqrt(d) and s2_j = (q2 . k2_j) / sqrt(d), d being the width of one
 *      query/key half  ([U] worked example: each query/key half is n x d and the scores are divided by sqrt(d)).
 *   3. Two softmax maps over J: a_j = exp(s1_j) / sum exp(s1), b_j likewise from s2  ([U] worked example).
 *      The row maximum is subtracted before exp; this changes no value in exact arithmetic.
 *   4. The difference map w_j = a_j - lambda * b_j  ([U] worked example; [J] main features).
 *   5. The output row o = sum_j w_j v_j, a 2d-wide vector (values are twice as wide: [U] worked example).
 *   6. layer == 0: o is the result (raw).  layer >= 1: per-head normalisation and output scale, [U] paragraph
 *      after the example: y = o / sqrt(mean_c(o_c^2) + 1e-5) * (1 - lambda_init(layer)), RMS normalisation over
 *      the head's 2d channels, eps 1e-5 inside the root, no affine; lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l-1)).
 *
 * Backward (oracle_diffattn_bwd): the gradients of a scalar loss with respect to q1, k1, q2, k2, v and lambda,
 * given the loss's gradient dy with respect to the output.  The pages give no backward pass; it is the chain rule
 * applied to steps 2-6 above, written out row by row (no blocking, no recomputation tricks):
 *   7. (layer >= 1) through y = g r o with r = (mean_c o_c^2 + 1e-5)^(-1/2):  do = g r dy - g r^3 o (dy . o) / 2d.
 *   8. o = o1 - lambda o2 with o1 = sum_j a_j v_j, o2 = sum_j b_j v_j:  dv_j += (a_j - lambda b_j) do,
 *      d(lambda) -= do . o2,  da_j = do . v_j,  db_j = -lambda do . v_j.
 *   9. Softmax:  ds1_j = a_j (da_j - sum_k a_k da_k),  ds2_j = b_j (db_j - sum_k b_k db_k).
 *  10. Scores s = q . k / sqrt(d):  dq_i += ds_j k_j / sqrt(d),  dk_j += ds_j q_i / sqrt(d), per map.
 *
 * Mutants: compiling with -DORACLE_MUTANT=k plants one deliberate mistake (k = 1..10 in the forward, 11..15 in
 * the backward, see the switch points below).  The test suite builds each mutant and checks that the pins catch
 * it.  The default build has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

int oracle_mutant(void) { return ORACLE_MUTANT; }

/* lambda_init(l) = 0.8 - 0.6 * exp(-0.3 * (l - 1)) for a 1-based layer index ([U] paragraph after the example). */
double oracle_lambda_init(int layer)
{
#if ORACLE_MUTANT == 1
    return 0.8 - 0.6 * exp(-0.3 * (double)layer);          /* mutant: 0-based layer */
#else
    return 0.8 - 0.6 * exp(-0.3 * (double)(layer - 1));
#endif
}

static int key_visible(int64_t i, int64_t j, int64_t Nq, int64_t Nk, int causal)
{
    if (!causal)
        return 1;
#if ORACLE_MUTANT == 2
    return j < i + (Nk - Nq);                              /* mutant: strict mask drops the diagonal */
#else
    return j <= i + (Nk - Nq);
#endif
}

/* Softmax of s[0..n-1] over the entries with vis[j] != 0, written to p (0 where not visible). */
static void softmax_visible(const double *s, const unsigned char *vis, int64_t n, double *p)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j)
        if (vis[j] && s[j] > m)
            m = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j)
#if ORACLE_MUTANT == 10
        z += exp(s[j] - m);                                /* mutant: masked keys kept in the denominator */
#else
        z += vis[j] ? exp(s[j] - m) : 0.0;
#endif
    for (int64_t j = 0; j < n; ++j)
        p[j] = vis[j] ? exp(s[j] - m) / z : 0.0;
}

static double dot(const float *a, const float *b, int64_t n)
{
    double acc = 0.0;
    for (int64_t t = 0; t < n; ++t)
        acc += (double)a[t] * (double)b[t];
    return acc;
}

/*
 * One query row of one head.  q1,q2: d floats; k1,k2: Nk x d; v: Nk x 2d (row-major).
 * scratch: 5*Nk doubles + Nk bytes.  out: 2d doubles.  w (optional): Nk doubles, the difference map row.
 */
static void diffattn_row(const float *q1, const float *q2, const float *k1, const float *k2, const float *v,
                         int64_t i, int64_t Nq, int64_t Nk, int64_t d, double lambda, int layer, int causal,
                         double *scratch, unsigned char *vis, double *out, double *w)
{
    double *s1 = scratch, *s2 = scratch + Nk, *a = scratch + 2 * Nk, *b = scratch + 3 * Nk, *wd = scratch + 4 * Nk;
    const int64_t dv = 2 * d;

    /* step 1: visible keys */
    for (int64_t j = 0; j < Nk; ++j)
        vis[j] = (unsigned char)key_visible(i, j, Nq, Nk, causal);

    /* step 2: scaled scores of both maps */
#if ORACLE_MUTANT == 3
    const double root_d = sqrt((double)dv);                /* mutant: full head width in the scale */
#elif ORACLE_MUTANT == 4
    const double root_d = 1.0;                             /* mutant: scale dropped (as one page writes it) */
#else
    const double root_d = sqrt((double)d);
#endif
    for (int64_t j = 0; j < Nk; ++j) {
#if ORACLE_MUTANT == 5
        s1[j] = dot(q1, k2 + j * d, d) / root_d;           /* mutant: maps' keys swapped */
        s2[j] = dot(q2, k1 + j * d, d) / root_d;
#else
        s1[j] = dot(q1, k1 + j * d, d) / root_d;
        s2[j] = dot(q2, k2 + j * d, d) / root_d;
#endif
    }

    /* step 3: the two softmax maps */
    softmax_visible(s1, vis, Nk, a);
    softmax_visible(s2, vis, Nk, b);

    /* step 4: difference map */
    for (int64_t j = 0; j < Nk; ++j)
#if ORACLE_MUTANT == 6
        wd[j] = a[j] + lambda * b[j];                      /* mutant: wrong sign */
#else
        wd[j] = a[j] - lambda * b[j];
#endif

    /* step 5: mix the 2d-wide values */
    for (int64_t c = 0; c < dv; ++c)
        out[c] = 0.0;
    for (int64_t j = 0; j < Nk; ++j) {
        if (!vis[j])
            continue;
        const float *vj = v + j * dv;
        for (int64_t c = 0; c < dv; ++c)
            out[c] += wd[j] * (double)vj[c];
    }

    /* step 6: per-head RMS normalisation and the (1 - lambda_init) scale */
    if (layer >= 1) {
        double ms = 0.0;
        for (int64_t c = 0; c < dv; ++c)
            ms += out[c] * out[c];
#if ORACLE_MUTANT == 9
        ms /= (double)d;                                   /* mutant: mean over half the channels' count */
#else
        ms /= (double)dv;
#endif
#if ORACLE_MUTANT == 7
        const double r = 1.0 / (sqrt(ms) + 1e-5);          /* mutant: eps outside the root */
#else
        const double r = 1.0 / sqrt(ms + 1e-5);
#endif
#if ORACLE_MUTANT == 8
        const double g = oracle_lambda_init(layer);        /* mutant: lambda_init instead of 1 - lambda_init */
#else
        const double g = 1.0 - oracle_lambda_init(layer);
#endif
        for (int64_t c = 0; c < dv; ++c)
            out[c] = out[c] * r * g;
    }
    if (w)
        memcpy(w, wd, (size_t)Nk * sizeof(double));
}

/*
 * Whole-problem entry point.
 *   q1,q2: [B][H][Nq][d] float32;  k1,k2: [B][H][Nk][d];  v: [B][H][Nk][2d]   (bf16 inputs arrive widened).
 *   rows:  indices into the flattened [B][H][Nq] query rows to evaluate, or NULL for all of them (nrows must
 *          then equal B*H*Nq).
 *   out:   nrows x 2d doubles.   diff: nrows x Nk doubles or NULL (entries of masked keys are 0).
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 for bad arguments.
 */
int oracle_diffattn(const float *q1, const float *k1, const float *q2, const float *k2, const float *v,
                    int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, double lambda, int layer, int causal,
                    const int64_t *rows, int64_t nrows, double *out, double *diff, int nthreads)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 1 || d < 1 || layer < 0 || nrows < 0 || !out)
        return -1;
    if (!rows && nrows != B * H * Nq)
        return -1;
    if (causal && Nq > Nk)
        return -1;
    const int64_t total = B * H * Nq;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= total)
            return -1;
    const int64_t dv = 2 * d;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *scratch = (double *)malloc((size_t)(5 * Nk) * sizeof(double));
        unsigned char *vis = (unsigned char *)malloc((size_t)Nk);
        if (!scratch || !vis) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 16)
#endif
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t flat = rows ? rows[r] : r;
                const int64_t bh = flat / Nq, i = flat % Nq;
                diffattn_row(q1 + flat * d, q2 + flat * d, k1 + bh * Nk * d, k2 + bh * Nk * d, v + bh * Nk * dv,
                             i, Nq, Nk, d, lambda, layer, causal, scratch, vis, out + r * dv,
                             diff ? diff + r * Nk : NULL);
            }
        }
        free(scratch);
        free(vis);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/*
 * Backward for a square problem (Nq = Nk = N), all rows.  Inputs as in oracle_diffattn plus dy: [B][H][N][2d]
 * float32 (the gradient of the loss with respect to the output).  lambda_heads: H doubles (lambda of head h).
 * Outputs (doubles, overwritten): dq1, dk1, dq2, dk2 [B][H][N][d]; dv [B][H][N][2d]; dlambda [H] (summed over
 * the batch).  Heads are independent, so OpenMP runs over (b, h); within a head the rows run in order, since
 * every row adds to the key-side gradients.  Returns 0, or -1 for bad arguments or memory.
 */
int oracle_diffattn_bwd(const float *q1, const float *k1, const float *q2, const float *k2, const float *v,
                        const float *dy, int64_t B, int64_t H, int64_t N, int64_t d, const double *lambda_heads,
                        int layer, int causal, double *dq1, double *dk1, double *dq2, double *dk2, double *dv,
                        double *dlambda, int nthreads)
{
    if (B < 0 || H < 0 || N < 1 || d < 1 || layer < 0 || !lambda_heads || !dq1 || !dk1 || !dq2 || !dk2 || !dv ||
        !dlambda)
        return -1;
    const int64_t dvw = 2 * d, BH = B * H;
    memset(dk1, 0, (size_t)(BH * N * d) * sizeof(double));
    memset(dk2, 0, (size_t)(BH * N * d) * sizeof(double));
    memset(dv, 0, (size_t)(BH * N * dvw) * sizeof(double));
    double *dl_bh = (double *)calloc((size_t)(BH > 0 ? BH : 1), sizeof(double));
    if (!dl_bh)
        return -1;
    const double root_d = sqrt((double)d);
    const double g = layer >= 1 ? 1.0 - oracle_lambda_init(layer) : 1.0;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *buf = (double *)malloc((size_t)(7 * N + 5 * dvw) * sizeof(double));
        unsigned char *vis = (unsigned char *)malloc((size_t)N);
        if (!buf || !vis) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        } else {
            double *s1 = buf, *s2 = buf + N, *a = buf + 2 * N, *b = buf + 3 * N, *da = buf + 4 * N;
            double *ds1 = buf + 5 * N, *ds2 = buf + 6 * N;
            double *o1 = buf + 7 * N, *o2 = o1 + dvw, *o = o2 + dvw, *dout = o + dvw;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t bh = 0; bh < BH; ++bh) {
                const double lambda = lambda_heads[bh % H];
                const float *K1 = k1 + bh * N * d, *K2 = k2 + bh * N * d, *V = v + bh * N * dvw;
                for (int64_t i = 0; i < N; ++i) {
                    const float *Q1 = q1 + (bh * N + i) * d, *Q2 = q2 + (bh * N + i) * d;
                    const float *DY = dy + (bh * N + i) * dvw;
                    /* forward quantities of row i (steps 1-5) */
                    for (int64_t j = 0; j < N; ++j) {
                        vis[j] = (unsigned char)key_visible(i, j, N, N, causal);
                        s1[j] = dot(Q1, K1 + j * d, d) / root_d;
                        s2[j] = dot(Q2, K2 + j * d, d) / root_d;
                    }
                    softmax_visible(s1, vis, N, a);
                    softmax_visible(s2, vis, N, b);
                    for (int64_t c = 0; c < dvw; ++c)
                        o1[c] = o2[c] = 0.0;
                    for (int64_t j = 0; j < N; ++j) {
                        if (!vis[j])
                            continue;
                        for (int64_t c = 0; c < dvw; ++c) {
                            o1[c] += a[j] * (double)V[j * dvw + c];
                            o2[c] += b[j] * (double)V[j * dvw + c];
                        }
                    }
                    for (int64_t c = 0; c < dvw; ++c)
                        o[c] = o1[c] - lambda * o2[c];
                    /* step 7: through the normalisation and scale */
                    if (layer >= 1) {
                        double ms = 0.0, dyo = 0.0;
                        for (int64_t c = 0; c < dvw; ++c) {
                            ms += o[c] * o[c];
                            dyo += (double)DY[c] * o[c];
                        }
                        const double r = 1.0 / sqrt(ms / (double)dvw + 1e-5);
                        for (int64_t c = 0; c < dvw; ++c)
#if ORACLE_MUTANT == 13
                            dout[c] = g * r * (double)DY[c];                       /* mutant: no projection term */
#else
                            dout[c] = g * r * (double)DY[c] - g * r * r * r * o[c] * dyo / (double)dvw;
#endif
                    } else {
                        for (int64_t c = 0; c < dvw; ++c)
                            dout[c] = (double)DY[c];
                    }
                    /* step 8: the difference of the maps, lambda and the values */
                    double dl = 0.0;
                    for (int64_t c = 0; c < dvw; ++c)
                        dl += dout[c] * o2[c];
#if ORACLE_MUTANT == 14
                    dl_bh[bh] += dl;                                                /* mutant: sign of d(lambda) */
#else
                    dl_bh[bh] -= dl;
#endif
                    double D1 = 0.0, D2 = 0.0;
                    for (int64_t j = 0; j < N; ++j) {
                        da[j] = 0.0;
                        if (!vis[j])
                            continue;
                        for (int64_t c = 0; c < dvw; ++c)
                            da[j] += dout[c] * (double)V[j * dvw + c];
                        D1 += a[j] * da[j];
                        D2 += b[j] * (-lambda * da[j]);
                        for (int64_t c = 0; c < dvw; ++c)
                            dv[(bh * N + j) * dvw + c] += (a[j] - lambda * b[j]) * dout[c];
                    }
                    /* step 9: the two softmaxes */
                    for (int64_t j = 0; j < N; ++j) {
#if ORACLE_MUTANT == 11
                        ds1[j] = a[j] * da[j];                                      /* mutant: row term dropped */
#else
                        ds1[j] = a[j] * (da[j] - D1);
#endif
#if ORACLE_MUTANT == 12
                        ds2[j] = b[j] * (da[j] - D2);                               /* mutant: -lambda missing */
#else
                        ds2[j] = b[j] * (-lambda * da[j] - D2);
#endif
                    }
                    /* step 10: the scores */
                    double *DQ1 = dq1 + (bh * N + i) * d, *DQ2 = dq2 + (bh * N + i) * d;
                    for (int64_t t = 0; t < d; ++t)
                        DQ1[t] = DQ2[t] = 0.0;
                    for (int64_t j = 0; j < N; ++j) {
                        if (!vis[j])
                            continue;
                        for (int64_t t = 0; t < d; ++t) {
                            DQ1[t] += ds1[j] * (double)K1[j * d + t] / root_d;
                            DQ2[t] += ds2[j] * (double)K2[j * d + t] / root_d;
#if ORACLE_MUTANT == 15
                            dk1[(bh * N + j) * d + t] += ds1[j] * (double)Q2[t] / root_d;  /* mutant: q of map 2 */
#else
                            dk1[(bh * N + j) * d + t] += ds1[j] * (double)Q1[t] / root_d;
#endif
                            dk2[(bh * N + j) * d + t] += ds2[j] * (double)Q2[t] / root_d;
                        }
                    }
                }
            }
        }
        free(buf);
        free(vis);
    }
    (void)nthreads;
    for (int64_t h = 0; h < H; ++h)
        dlambda[h] = 0.0;
    for (int64_t bh = 0; bh < BH; ++bh)
        dlambda[bh % H] += dl_bh[bh];
    free(dl_bh);
    return bad ? -1 : 0;
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
