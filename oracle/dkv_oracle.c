/*
 * dkv_oracle.c -- CPU oracle for DualKV shared-prompt attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path loads this library; only
 * tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg do.  It shares no
 * code, header, table or helper with the HIP path.
 *
 * What it computes: plain causal softmax attention of ONE sequence, in double
 * precision, which is the per-sequence attention of the N-copy packing defined in
 * "DualKV: Shared-Prompt Flash Attention for Efficient RL Training with Large
 * Rollouts and Long Contexts" (arXiv 2605.15422), §2.1 "Baseline: standard packing
 * with replicated prompts", eq. (2):
 *
 *     O = softmax(scale * Q K^T + M_causal) V,          scale = 1/sqrt(d) by default
 *
 * and its gradients with respect to Q, K and V for an upstream gradient dO (the
 * chain rule through the row softmax; the paper states which gradients the
 * backward returns in §3.2 and Appendix A.4 but prints no formulas for them).
 * The N-copy packing, the per-copy sums of eq. (6) and the comparison layout are
 * assembled by the Python wrapper in oracle/__init__.py.
 *
 * Readings of points the paper leaves open:
 *   - window_left = -1 is global causal; otherwise key j is visible from query t
 *     iff t - window_left <= j <= t (the paper's kernel-native causal sliding
 *     window, §3, is only said to equal windowed FlashAttention-2).
 *   - GQA: q-head h reads kv-head kvh[h] (contiguous groups by default, §4.1
 *     "GQA 4:1").
 *   - LSE is the natural-log log-sum-exp of the scaled logits of each row.
 *
 * Storage: row-major [S, H, d] double arrays for one sequence of S tokens.
 * Every sum and dot product is accumulated in double.  Functions return 0 on
 * success and a negative value on an invalid argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* First and last visible key of query position t. */
static void visible_range(int t, int window_left, int *j0, int *j1)
{
    int lo = 0;
    if (window_left >= 0 && t - window_left > 0)
        lo = t - window_left;
    *j0 = lo;
    *j1 = t;
}

static double dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int c = 0; c < d; ++c)
        s += a[c] * b[c];
    return s;
}

static int check_args(int S, int Hq, int Hkv, int d, const int *kvh)
{
    if (S < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || kvh == NULL)
        return -1;
    for (int h = 0; h < Hq; ++h)
        if (kvh[h] < 0 || kvh[h] >= Hkv)
            return -2;
    return 0;
}

/*
 * Softmax weights of row (t, h): p[j - j0] = exp(s_j) / sum_j' exp(s_j') over the
 * visible keys, with s_j = scale * <q_t,h , k_j,kvh[h]>.  Returns the log-sum-exp.
 * The maximum is subtracted before exponentiating (the same value, computed
 * without overflow).
 */
static double row_softmax(int t, int h, int Hq, int Hkv, int d, const int *kvh,
                          int window_left, double scale, const double *q,
                          const double *k, double *p, int *j0_out, int *cnt_out)
{
    int j0, j1;
    visible_range(t, window_left, &j0, &j1);
    int cnt = j1 - j0 + 1;
    const double *qt = q + ((size_t)t * Hq + h) * d;
    int g = kvh[h];
    double m = -INFINITY;
    for (int j = j0; j <= j1; ++j) {
        double s = scale * dot(qt, k + ((size_t)j * Hkv + g) * d, d);
        p[j - j0] = s;
        if (s > m)
            m = s;
    }
    double l = 0.0;
    for (int n = 0; n < cnt; ++n)
        l += exp(p[n] - m);
    for (int n = 0; n < cnt; ++n)
        p[n] = exp(p[n] - m) / l;
    *j0_out = j0;
    *cnt_out = cnt;
    return m + log(l);
}

/*
 * Forward rows: for each selected query position tsel[n] and every q-head h,
 *   o[n, h, :] = sum_j p_j v_j,  lse[n, h] = log sum_j exp(s_j).
 */
int oracle_fwd_rows(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                    double scale, const double *q, const double *k, const double *v,
                    int nsel, const int *tsel, double *o, double *lse)
{
    int rc = check_args(S, Hq, Hkv, d, kvh);
    if (rc)
        return rc;
    for (int n = 0; n < nsel; ++n)
        if (tsel[n] < 0 || tsel[n] >= S)
            return -3;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < nsel; ++n)
        for (int h = 0; h < Hq; ++h) {
            int t = tsel[n];
            double *p = (double *)malloc(sizeof(double) * (size_t)(t + 1));
            if (!p) {
                bad = 1;
                continue;
            }
            int j0, cnt;
            double L = row_softmax(t, h, Hq, Hkv, d, kvh, window_left, scale, q, k, p,
                                   &j0, &cnt);
            double *ot = o + ((size_t)n * Hq + h) * d;
            const int g = kvh[h];
            for (int c = 0; c < d; ++c)
                ot[c] = 0.0;
            for (int i = 0; i < cnt; ++i) {
                const double *vj = v + ((size_t)(j0 + i) * Hkv + g) * d;
                for (int c = 0; c < d; ++c)
                    ot[c] += p[i] * vj[c];
            }
            lse[(size_t)n * Hq + h] = L;
            free(p);
        }
    return bad ? -4 : 0;
}

/*
 * Backward, row-local part: for each selected query position tsel[n] and q-head h,
 *   dP_j   = <dO_t, v_j>
 *   delta  = sum_j p_j dP_j                      (softmax Jacobian term)
 *   dS_j   = p_j (dP_j - delta)
 *   dq     = scale * sum_j dS_j k_j
 * Also returns the row's lse and delta, which the key-side part needs.
 */
int oracle_bwd_rows(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                    double scale, const double *q, const double *k, const double *v,
                    const double *dout, int nsel, const int *tsel, double *dq,
                    double *lse, double *delta)
{
    int rc = check_args(S, Hq, Hkv, d, kvh);
    if (rc)
        return rc;
    for (int n = 0; n < nsel; ++n)
        if (tsel[n] < 0 || tsel[n] >= S)
            return -3;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < nsel; ++n)
        for (int h = 0; h < Hq; ++h) {
            int t = tsel[n];
            double *p = (double *)malloc(sizeof(double) * 2 * (size_t)(t + 1));
            if (!p) {
                bad = 1;
                continue;
            }
            double *dp = p + (t + 1);
            int j0, cnt;
            double L = row_softmax(t, h, Hq, Hkv, d, kvh, window_left, scale, q, k, p,
                                   &j0, &cnt);
            const int g = kvh[h];
            const double *dot_ = dout + ((size_t)t * Hq + h) * d;
            double D = 0.0;
            for (int i = 0; i < cnt; ++i) {
                dp[i] = dot(dot_, v + ((size_t)(j0 + i) * Hkv + g) * d, d);
                D += p[i] * dp[i];
            }
            double *dqt = dq + ((size_t)n * Hq + h) * d;
            for (int c = 0; c < d; ++c)
                dqt[c] = 0.0;
            for (int i = 0; i < cnt; ++i) {
                double ds = p[i] * (dp[i] - D);
                const double *kj = k + ((size_t)(j0 + i) * Hkv + g) * d;
                for (int c = 0; c < d; ++c)
                    dqt[c] += scale * ds * kj[c];
            }
            lse[(size_t)n * Hq + h] = L;
            delta[(size_t)n * Hq + h] = D;
            free(p);
        }
    return bad ? -4 : 0;
}

/*
 * Backward, key-side part: for each selected key position jsel[n] and kv-head g,
 *   dk = scale * sum_{t sees j} sum_{h: kvh[h] = g} dS_tj q_t,h
 *   dv =         sum_{t sees j} sum_{h: kvh[h] = g} p_tj  dO_t,h
 * with p_tj = exp(s_tj - lse_t,h) and dS_tj = p_tj (<dO_t,h, v_j> - delta_t,h).
 * lse and delta are [S, Hq] arrays for every query position (from
 * oracle_bwd_rows over all rows).
 */
int oracle_bwd_keys(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                    double scale, const double *q, const double *k, const double *v,
                    const double *dout, const double *lse, const double *delta,
                    int nsel, const int *jsel, double *dk, double *dv)
{
    int rc = check_args(S, Hq, Hkv, d, kvh);
    if (rc)
        return rc;
    for (int n = 0; n < nsel; ++n)
        if (jsel[n] < 0 || jsel[n] >= S)
            return -3;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < nsel; ++n)
        for (int g = 0; g < Hkv; ++g) {
            int j = jsel[n];
            const double *kj = k + ((size_t)j * Hkv + g) * d;
            const double *vj = v + ((size_t)j * Hkv + g) * d;
            double *dkj = dk + ((size_t)n * Hkv + g) * d;
            double *dvj = dv + ((size_t)n * Hkv + g) * d;
            for (int c = 0; c < d; ++c) {
                dkj[c] = 0.0;
                dvj[c] = 0.0;
            }
            for (int t = j; t < S; ++t) {
                int j0, j1;
                visible_range(t, window_left, &j0, &j1);
                if (j < j0)
                    continue;
                for (int h = 0; h < Hq; ++h) {
                    if (kvh[h] != g)
                        continue;
                    const double *qt = q + ((size_t)t * Hq + h) * d;
                    const double *dot_ = dout + ((size_t)t * Hq + h) * d;
                    double s = scale * dot(qt, kj, d);
                    double p = exp(s - lse[(size_t)t * Hq + h]);
                    double ds = p * (dot(dot_, vj, d) - delta[(size_t)t * Hq + h]);
                    for (int c = 0; c < d; ++c) {
                        dkj[c] += scale * ds * qt[c];
                        dvj[c] += p * dot_[c];
                    }
                }
            }
        }
    return 0;
}

/*
 * Backward contributions of a few query rows, for an upstream gradient that is zero
 * on every other row.  For each selected row tsel[n] (its query q_sel[n] and
 * upstream gradient dout_sel[n], [nsel, Hq, d]) and q-head h, over the visible keys
 * j of that row in a sequence with keys k / values v ([S, Hkv, d]):
 *   p_j = softmax_j(scale <q, k_j>),  dP_j = <dO, v_j>,  delta = sum_j p_j dP_j,
 *   dS_j = p_j (dP_j - delta)
 *   dq[n, h]        = scale * sum_j dS_j k_j        (written)
 *   dk[j, kvh[h]]  += scale * dS_j q                (added)
 *   dv[j, kvh[h]]  += p_j dO                         (added)
 * The same chain rule as oracle_bwd_rows / oracle_bwd_keys, restricted to the rows
 * whose upstream gradient is non-zero (rows with dO = 0 add nothing).  Rows are taken
 * one at a time; the keys of a row are split over threads, so no two threads add to
 * the same key.
 */
int oracle_bwd_scatter(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                       double scale, const double *k, const double *v, int nsel,
                       const int *tsel, const double *q_sel, const double *dout_sel,
                       double *dq, double *dk, double *dv)
{
    int rc = check_args(S, Hq, Hkv, d, kvh);
    if (rc)
        return rc;
    for (int n = 0; n < nsel; ++n)
        if (tsel[n] < 0 || tsel[n] >= S)
            return -3;
    double *s = (double *)malloc(sizeof(double) * 2 * (size_t)(S > 0 ? S : 1));
    if (!s)
        return -4;
    double *dp = s + S;
    for (int n = 0; n < nsel; ++n) {
        const int t = tsel[n];
        int j0, j1;
        visible_range(t, window_left, &j0, &j1);
        const int cnt = j1 - j0 + 1;
        for (int h = 0; h < Hq; ++h) {
            const int g = kvh[h];
            const double *qt = q_sel + ((size_t)n * Hq + h) * d;
            const double *dot_ = dout_sel + ((size_t)n * Hq + h) * d;
#pragma omp parallel for schedule(static)
            for (int i = 0; i < cnt; ++i) {
                s[i] = scale * dot(qt, k + ((size_t)(j0 + i) * Hkv + g) * d, d);
                dp[i] = dot(dot_, v + ((size_t)(j0 + i) * Hkv + g) * d, d);
            }
            double m = -INFINITY;
            for (int i = 0; i < cnt; ++i)
                if (s[i] > m)
                    m = s[i];
            double l = 0.0;
            for (int i = 0; i < cnt; ++i)
                l += exp(s[i] - m);
            double delta = 0.0;
            for (int i = 0; i < cnt; ++i) {
                s[i] = exp(s[i] - m) / l;          /* p_j */
                delta += s[i] * dp[i];
            }
            double *dqt = dq + ((size_t)n * Hq + h) * d;
            for (int c = 0; c < d; ++c)
                dqt[c] = 0.0;
            for (int i = 0; i < cnt; ++i) {
                const double ds = s[i] * (dp[i] - delta);
                const double *kj = k + ((size_t)(j0 + i) * Hkv + g) * d;
                for (int c = 0; c < d; ++c)
                    dqt[c] += scale * ds * kj[c];
            }
#pragma omp parallel for schedule(static)
            for (int i = 0; i < cnt; ++i) {
                const double ds = s[i] * (dp[i] - delta);
                double *dkj = dk + ((size_t)(j0 + i) * Hkv + g) * d;
                double *dvj = dv + ((size_t)(j0 + i) * Hkv + g) * d;
                for (int c = 0; c < d; ++c) {
                    dkj[c] += scale * ds * qt[c];
                    dvj[c] += s[i] * dot_[c];
                }
            }
        }
    }
    free(s);
    return 0;
}

/*
 * Forward rows as oracle_fwd_rows, with the queries of the selected rows given on
 * their own (q_sel [nsel, Hq, d]) so that long sequences need not be materialized:
 * row n sits at position tsel[n] of a sequence with keys k / values v [S, Hkv, d].
 */
int oracle_fwd_sel(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                   double scale, const double *k, const double *v, int nsel,
                   const int *tsel, const double *q_sel, double *o, double *lse)
{
    int rc = check_args(S, Hq, Hkv, d, kvh);
    if (rc)
        return rc;
    for (int n = 0; n < nsel; ++n)
        if (tsel[n] < 0 || tsel[n] >= S)
            return -3;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int n = 0; n < nsel; ++n)
        for (int h = 0; h < Hq; ++h) {
            const int t = tsel[n];
            double *p = (double *)malloc(sizeof(double) * (size_t)(t + 1));
            if (!p) {
                bad = 1;
                continue;
            }
            int j0, j1;
            visible_range(t, window_left, &j0, &j1);
            const int cnt = j1 - j0 + 1, g = kvh[h];
            const double *qt = q_sel + ((size_t)n * Hq + h) * d;
            double m = -INFINITY;
            for (int i = 0; i < cnt; ++i) {
                p[i] = scale * dot(qt, k + ((size_t)(j0 + i) * Hkv + g) * d, d);
                if (p[i] > m)
                    m = p[i];
            }
            double l = 0.0;
            for (int i = 0; i < cnt; ++i)
                l += exp(p[i] - m);
            double *ot = o + ((size_t)n * Hq + h) * d;
            for (int c = 0; c < d; ++c)
                ot[c] = 0.0;
            for (int i = 0; i < cnt; ++i) {
                const double w = exp(p[i] - m) / l;
                const double *vj = v + ((size_t)(j0 + i) * Hkv + g) * d;
                for (int c = 0; c < d; ++c)
                    ot[c] += w * vj[c];
            }
            lse[(size_t)n * Hq + h] = m + log(l);
            free(p);
        }
    return bad ? -4 : 0;
}
