/*
 * abi_consumer.c -- one DualKV training step driven from C through libdkv's C ABI alone
 * (include/dkv.h plus the HIP runtime for device memory and a stream; no Python, no
 * torch), with every output checked against the CPU oracle (oracle/liboracle.so).
 *
 * TEST INFRASTRUCTURE: it links the oracle, which nothing in the product path does.
 *
 * The step is the two-call decomposition of "DualKV: Shared-Prompt Flash Attention for
 * Efficient RL Training with Large Rollouts and Long Contexts" (arXiv 2605.15422), §2.2:
 * Call 1 over the single prompt copy (eq. (3)), Call 2 over the responses against the
 * shared prompt keys and their own (eq. (4), §3.1), and the backward with the prompt
 * keys' gradient of eq. (6) summed in one fp32 accumulator by both calls and cast once
 * (§3.2).  The oracle computes the N-copy packing's attention (§2.1, eq. (2)) sequence
 * by sequence; each copy's prompt rows get the upstream gradient dO_P / N (any split that
 * sums to dO_P is valid, App. A.5), and the prompt's gradients are the sums over copies.
 *
 * Usage: abi_consumer WINDOW_LEFT DTYPE HEADMAP
 *   WINDOW_LEFT  -1 (global causal) or w >= 0
 *   DTYPE        0 bf16, 1 fp32 (dkv_dtype)
 *   HEADMAP      0: contiguous GQA groups (kv_head_of_q NULL); 1: a permuted map
 * Prints one line per tensor; exits 0 when every tensor is within its bound, 1 on a
 * mismatch, 2 on a failed call.  Bounds: fp32 max|err| <= 1e-5; bf16 max|err| <=
 * 2e-2 max|ref| per tensor (LSE: 2e-3 absolute).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dkv.h"

/* oracle/liboracle.so (double precision, one sequence, row-major [S, H, d]) */
int oracle_fwd_rows(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                    double scale, const double *q, const double *k, const double *v,
                    int nsel, const int *tsel, double *o, double *lse);
int oracle_bwd_rows(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                    double scale, const double *q, const double *k, const double *v,
                    const double *dout, int nsel, const int *tsel, double *dq,
                    double *lse, double *delta);
int oracle_bwd_keys(int S, int Hq, int Hkv, int d, const int *kvh, int window_left,
                    double scale, const double *q, const double *k, const double *v,
                    const double *dout, const double *lse, const double *delta,
                    int nsel, const int *jsel, double *dk, double *dv);

enum { P = 70, N = 3, HQ = 4, HKV = 2, D = 128 };
static const int kLens[N] = {45, 0, 33};

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));     \
            exit(2);                                                           \
        }                                                                      \
    } while (0)
#define DKV_OK_(x)                                                             \
    do {                                                                       \
        dkv_status s_ = (x);                                                   \
        if (s_ != DKV_OK) {                                                    \
            fprintf(stderr, "%s -> %d: %s\n", #x, (int)s_, dkv_last_error());  \
            exit(2);                                                           \
        }                                                                      \
    } while (0)

/* splitmix64: the test's own input stream (unit-variance uniform values) */
static uint64_t g_state = 0x9e3779b97f4a7c15ull;
static double next_uniform(void)
{
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return ((double)(z >> 11) / 9007199254740992.0 * 2.0 - 1.0) * 1.7320508075688772;
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float x)
{
    uint32_t b;
    memcpy(&b, &x, 4);
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}
static float from_bf16(uint16_t h)
{
    uint32_t b = (uint32_t)h << 16;
    float x;
    memcpy(&x, &b, 4);
    return x;
}

static int g_bf16;   /* element type of the tensors */

/* n values of the stream, rounded to the tensor type (the same values feed both sides) */
static double *draw(size_t n)
{
    double *x = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) {
        float f = (float)next_uniform();
        x[i] = g_bf16 ? (double)from_bf16(to_bf16(f)) : (double)f;
    }
    return x;
}
static size_t esize(void) { return g_bf16 ? 2 : 4; }
static void *to_device(const double *x, size_t n)
{
    void *h = malloc(n * esize() + 1), *dptr = NULL;
    for (size_t i = 0; i < n; ++i) {
        if (g_bf16)
            ((uint16_t *)h)[i] = to_bf16((float)x[i]);
        else
            ((float *)h)[i] = (float)x[i];
    }
    HIP_OK(hipMalloc(&dptr, n * esize() + 16));
    HIP_OK(hipMemcpy(dptr, h, n * esize(), hipMemcpyHostToDevice));
    free(h);
    return dptr;
}
static void *dev_alloc(size_t bytes)
{
    void *p = NULL;
    HIP_OK(hipMalloc(&p, bytes + 16));
    return p;
}
static double *from_device(const void *dptr, size_t n, int is_f32)
{
    const size_t es = is_f32 ? 4 : esize();
    void *h = malloc(n * es + 1);
    double *x = malloc(n * sizeof(double) + 1);
    HIP_OK(hipMemcpy(h, dptr, n * es, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < n; ++i)
        x[i] = (es == 2) ? (double)from_bf16(((uint16_t *)h)[i]) : (double)((float *)h)[i];
    free(h);
    return x;
}

static int g_fail;
static void compare(const char *name, const double *got, const double *ref, size_t n,
                    int is_lse)
{
    double err = 0.0, mref = 0.0;
    int finite = 1;
    for (size_t i = 0; i < n; ++i) {
        if (!isfinite(got[i]))
            finite = 0;
        err = fmax(err, fabs(got[i] - ref[i]));
        mref = fmax(mref, fabs(ref[i]));
    }
    double bound = !g_bf16 ? 1e-5 : is_lse ? 2e-3 : (mref > 0 ? 2e-2 * mref : 1e-4);
    int ok = finite && err <= bound;
    printf("%-6s max|err| %.3e  bound %.3e  %s\n", name, err, bound, ok ? "ok" : "FAIL");
    if (!ok)
        g_fail = 1;
}

int main(int argc, char **argv)
{
    if (argc != 4) {
        fprintf(stderr, "usage: %s WINDOW_LEFT DTYPE HEADMAP\n", argv[0]);
        return 2;
    }
    const int wl = atoi(argv[1]);
    const int dtype = atoi(argv[2]);
    const int headmap = atoi(argv[3]);
    if (dtype != DKV_BF16 && dtype != DKV_FP32)
        return 2;
    g_bf16 = dtype == DKV_BF16;
    printf("abi_consumer: P=%d N=%d lens={%d,%d,%d} Hq=%d Hkv=%d d=%d window_left=%d %s %s\n",
           P, N, kLens[0], kLens[1], kLens[2], HQ, HKV, D, wl, g_bf16 ? "bf16" : "fp32",
           headmap ? "permuted head map" : "contiguous heads");
    fflush(stdout);

    int cu[N + 1] = {0};
    for (int i = 0; i < N; ++i)
        cu[i + 1] = cu[i] + kLens[i];
    const int T = cu[N];
    const int cu_p[2] = {0, P};
    /* GQA map: q-head h reads kv head kvh[h]; each kv head serves HQ / HKV q-heads */
    int kvh[HQ];
    static const int kPermuted[HQ] = {1, 0, 0, 1};
    for (int h = 0; h < HQ; ++h)
        kvh[h] = headmap ? kPermuted[h] : h / (HQ / HKV);

    const size_t nqp = (size_t)P * HQ * D, nkp = (size_t)P * HKV * D;
    const size_t nqr = (size_t)T * HQ * D, nkr = (size_t)T * HKV * D;
    double *q_p = draw(nqp), *k_p = draw(nkp), *v_p = draw(nkp);
    double *q_r = draw(nqr), *k_r = draw(nkr), *v_r = draw(nkr);
    double *do_p = draw(nqp), *do_r = draw(nqr);

    /* ---- the library: one step through the C ABI ---- */
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    dkv_params p1, p2;
    memset(&p1, 0, sizeof p1);
    p1.num_seqs = 1;
    p1.ctx_len = 0;
    p1.num_heads_q = HQ;
    p1.num_heads_kv = HKV;
    p1.head_dim = D;
    p1.window_left = wl;
    p1.softmax_scale = 0.f;
    p1.dtype = dtype;
    p1.cu_seqlens_host = cu_p;
    p1.kv_head_of_q = headmap ? kvh : NULL;
    p2 = p1;
    p2.num_seqs = N;
    p2.ctx_len = P;
    p2.cu_seqlens_host = cu;

    size_t ws_bytes = 0;
    const dkv_params *pc[4] = {&p1, &p2, &p1, &p2};
    const int calls[4] = {DKV_CALL_CTX_FWD, DKV_CALL_FWD, DKV_CALL_CTX_BWD, DKV_CALL_BWD};
    for (int c = 0; c < 4; ++c) {
        size_t b = dkv_workspace_size(pc[c], calls[c]);
        if (b > ws_bytes)
            ws_bytes = b;
    }
    void *ws = dev_alloc(ws_bytes);

    void *dq_p_in = to_device(q_p, nqp), *dk_p_in = to_device(k_p, nkp),
         *dv_p_in = to_device(v_p, nkp);
    void *dq_r_in = to_device(q_r, nqr), *dk_r_in = to_device(k_r, nkr),
         *dv_r_in = to_device(v_r, nkr);
    void *ddo_p = to_device(do_p, nqp), *ddo_r = to_device(do_r, nqr);
    const size_t es = esize();
    void *o_p = dev_alloc(nqp * es), *o_r = dev_alloc(nqr * es);
    float *lse_p = dev_alloc((size_t)HQ * P * 4), *lse_r = dev_alloc((size_t)HQ * T * 4);
    void *gq_p = dev_alloc(nqp * es), *gk_p = dev_alloc(nkp * es), *gv_p = dev_alloc(nkp * es);
    void *gq_r = dev_alloc(nqr * es), *gk_r = dev_alloc(nkr * es), *gv_r = dev_alloc(nkr * es);
    float *acc_dk = dev_alloc(nkp * 4), *acc_dv = dev_alloc(nkp * 4);

    DKV_OK_(dkv_ctx_fwd(&p1, dq_p_in, dk_p_in, dv_p_in, o_p, lse_p, ws, ws_bytes, stream));
    DKV_OK_(dkv_fwd(&p2, dq_r_in, dk_p_in, dv_p_in, dk_r_in, dv_r_in, o_r, lse_r, ws,
                    ws_bytes, stream));
    DKV_OK_(dkv_ctx_bwd(&p1, dq_p_in, dk_p_in, dv_p_in, o_p, lse_p, ddo_p, gq_p, NULL, NULL,
                        acc_dk, acc_dv, DKV_ACC_ZERO, ws, ws_bytes, stream));
    DKV_OK_(dkv_bwd(&p2, dq_r_in, dk_p_in, dv_p_in, dk_r_in, dv_r_in, o_r, lse_r, ddo_r, gq_r,
                    gk_r, gv_r, acc_dk, acc_dv, DKV_ACC_FINALIZE, gk_p, gv_p, ws, ws_bytes,
                    stream));
    HIP_OK(hipStreamSynchronize(stream));
    printf("abi_consumer: library step done\n");
    fflush(stdout);

    /* ---- the oracle: the N-copy packing, one copy at a time ---- */
    const double scale = 1.0 / sqrt((double)D);
    double *r_op = calloc(nqp, sizeof(double)), *r_lsep = calloc((size_t)HQ * P, sizeof(double));
    double *r_or = calloc(nqr + 1, sizeof(double)), *r_lser = calloc((size_t)HQ * T + 1, sizeof(double));
    double *r_dqp = calloc(nqp, sizeof(double)), *r_dkp = calloc(nkp, sizeof(double)),
           *r_dvp = calloc(nkp, sizeof(double));
    double *r_dqr = calloc(nqr + 1, sizeof(double)), *r_dkr = calloc(nkr + 1, sizeof(double)),
           *r_dvr = calloc(nkr + 1, sizeof(double));
    for (int i = 0; i < N; ++i) {
        const int R = kLens[i], S = P + R;
        const size_t qrow = (size_t)HQ * D, krow = (size_t)HKV * D;
        double *q = malloc(S * qrow * sizeof(double)), *k = malloc(S * krow * sizeof(double));
        double *v = malloc(S * krow * sizeof(double)), *dout = malloc(S * qrow * sizeof(double));
        memcpy(q, q_p, nqp * sizeof(double));
        memcpy(q + P * qrow, q_r + cu[i] * qrow, R * qrow * sizeof(double));
        memcpy(k, k_p, nkp * sizeof(double));
        memcpy(k + P * krow, k_r + cu[i] * krow, R * krow * sizeof(double));
        memcpy(v, v_p, nkp * sizeof(double));
        memcpy(v + P * krow, v_r + cu[i] * krow, R * krow * sizeof(double));
        for (size_t e = 0; e < nqp; ++e)
            dout[e] = do_p[e] / N;
        memcpy(dout + P * qrow, do_r + cu[i] * qrow, R * qrow * sizeof(double));

        int *sel = malloc(S * sizeof(int));
        for (int t = 0; t < S; ++t)
            sel[t] = t;
        double *o = malloc(S * qrow * sizeof(double)), *lse = malloc((size_t)S * HQ * sizeof(double));
        double *dq = malloc(S * qrow * sizeof(double)), *lse2 = malloc((size_t)S * HQ * sizeof(double));
        double *delta = malloc((size_t)S * HQ * sizeof(double));
        double *dk = malloc(S * krow * sizeof(double)), *dv = malloc(S * krow * sizeof(double));
        if (oracle_fwd_rows(S, HQ, HKV, D, kvh, wl, scale, q, k, v, S, sel, o, lse) ||
            oracle_bwd_rows(S, HQ, HKV, D, kvh, wl, scale, q, k, v, dout, S, sel, dq, lse2,
                            delta) ||
            oracle_bwd_keys(S, HQ, HKV, D, kvh, wl, scale, q, k, v, dout, lse2, delta, S, sel,
                            dk, dv)) {
            fprintf(stderr, "oracle call failed\n");
            return 2;
        }
        /* every copy's prompt rows hold the same O and LSE (App. A.2): take copy 0's */
        if (i == 0) {
            memcpy(r_op, o, nqp * sizeof(double));
            for (int t = 0; t < P; ++t)
                for (int h = 0; h < HQ; ++h)
                    r_lsep[(size_t)h * P + t] = lse[(size_t)t * HQ + h];
        }
        memcpy(r_or + cu[i] * qrow, o + P * qrow, R * qrow * sizeof(double));
        for (int t = 0; t < R; ++t)
            for (int h = 0; h < HQ; ++h)
                r_lser[(size_t)h * T + cu[i] + t] = lse[(size_t)(P + t) * HQ + h];
        /* the prompt's gradients are the sums over the copies (App. A.5, eq. (6)) */
        for (size_t e = 0; e < nqp; ++e)
            r_dqp[e] += dq[e];
        for (size_t e = 0; e < nkp; ++e) {
            r_dkp[e] += dk[e];
            r_dvp[e] += dv[e];
        }
        memcpy(r_dqr + cu[i] * qrow, dq + P * qrow, R * qrow * sizeof(double));
        memcpy(r_dkr + cu[i] * krow, dk + P * krow, R * krow * sizeof(double));
        memcpy(r_dvr + cu[i] * krow, dv + P * krow, R * krow * sizeof(double));
        free(q); free(k); free(v); free(dout); free(sel); free(o); free(lse); free(dq);
        free(lse2); free(delta); free(dk); free(dv);
    }

    compare("o_p", from_device(o_p, nqp, 0), r_op, nqp, 0);
    compare("lse_p", from_device(lse_p, (size_t)HQ * P, 1), r_lsep, (size_t)HQ * P, 1);
    compare("o_r", from_device(o_r, nqr, 0), r_or, nqr, 0);
    compare("lse_r", from_device(lse_r, (size_t)HQ * T, 1), r_lser, (size_t)HQ * T, 1);
    compare("dq_p", from_device(gq_p, nqp, 0), r_dqp, nqp, 0);
    compare("dk_p", from_device(gk_p, nkp, 0), r_dkp, nkp, 0);
    compare("dv_p", from_device(gv_p, nkp, 0), r_dvp, nkp, 0);
    compare("dq_r", from_device(gq_r, nqr, 0), r_dqr, nqr, 0);
    compare("dk_r", from_device(gk_r, nkr, 0), r_dkr, nkr, 0);
    compare("dv_r", from_device(gv_r, nkr, 0), r_dvr, nkr, 0);
    printf("abi_consumer: %s\n", g_fail ? "MISMATCH" : "all tensors within bound");
    return g_fail ? 1 : 0;
}
