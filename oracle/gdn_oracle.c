/*
 * gdn_oracle.c -- fp64 CPU oracle for the Gated DeltaNet mixer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code, header
 * or constant with the HIP library: it is the plain definition written out so
 * that the GPU results can be checked against it.
 *
 * What it computes (Atomic-GDN2 model card, section 2.1 "Gated DeltaNet-2"):
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 * with S_t a d_k x d_v matrix, alpha_t = exp(g_t) (the kernel receives the
 * log-decay g and exponentiates it itself, same section), and alpha_t either a
 * scalar per head-token (the scalar retention gate of Gated DeltaNet) or a
 * vector over the key channels (the per-key-channel gate of GDN-2 / KDA; the
 * MindPattern "Gated DeltaNet" page, finding of 2026-07-29 on the derivation
 * from softmax attention to KDA).
 *
 * The update is evaluated in its rank-1 form, which is the same matrix:
 *   S <- Diag(alpha) S                 (row c of S scaled by alpha_c: the
 *                                        decay acts on the key index, since
 *                                        k v^T puts keys on the rows)
 *   u <- S^T k                          (what the memory currently returns
 *                                        for key k)
 *   S <- S + beta k (v - u)^T           (delta rule: store the correction
 *                                        v - u, not v itself)
 *   o <- S^T q                          (read after the write)
 * Expanding: (I - beta k k^T) Diag(alpha) S + beta k v^T
 *          = Diag(alpha) S - beta k (k^T Diag(alpha) S) + beta k v^T.
 *
 * Readings where the pages are silent:
 *   - no 1/sqrt(d_k) scale on q: o = S^T q exactly as printed;
 *   - q and k normalisation, sigmoid on beta and the softplus clamp on g all
 *     happen before the call; the oracle takes q, k, v, g, beta as given;
 *   - everything is evaluated in double precision from the stored inputs
 *     (bf16 and fp32 inputs are passed as exactly upcast float values).
 *
 * Layouts (row-major, last index fastest):
 *   q, k  [B, T, H, K]     v [B, T, H, V]     beta [B, T, H]
 *   g     [B, T, H] (scalar gate) or [B, T, H, K] (channel gate)
 *   S0    [B, H, K, V] (float, may be NULL = zeros)
 *   o     [B, T, H, V] (double, may be NULL)   S_T [B, H, K, V] (double)
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/*
 * One independent (batch, head) slice: T sequential token updates.
 * Token t of each input starts at ptr + t * stride (elements); the channel
 * index is contiguous.  S holds the K x V state in and out (row-major).
 * o may be NULL.  work must hold K + V doubles.  Returns 0, or -1 on bad
 * arguments.
 */
int gdn_oracle_slice(int T, int K, int V, int channel_gate,
                     const float *q, long q_stride,
                     const float *k, long k_stride,
                     const float *v, long v_stride,
                     const float *g, long g_stride,
                     const float *beta, long beta_stride,
                     double *S, double *o, long o_stride)
{
    if (T < 0 || K <= 0 || V <= 0 || !q || !k || !v || !g || !beta || !S)
        return -1;
    double *alpha = (double *)malloc(sizeof(double) * (size_t)K);
    double *u = (double *)malloc(sizeof(double) * (size_t)V);
    if (!alpha || !u) {
        free(alpha);
        free(u);
        return -1;
    }
    for (int t = 0; t < T; ++t) {
        const float *qt = q + (long)t * q_stride;
        const float *kt = k + (long)t * k_stride;
        const float *vt = v + (long)t * v_stride;
        const float *gt = g + (long)t * g_stride;
        const double b = (double)beta[(long)t * beta_stride];

        /* alpha = exp(g): one value for the head, or one per key channel */
        for (int c = 0; c < K; ++c)
            alpha[c] = exp((double)(channel_gate ? gt[c] : gt[0]));

        /* S <- Diag(alpha) S */
        for (int c = 0; c < K; ++c) {
            double *row = S + (size_t)c * V;
            for (int j = 0; j < V; ++j)
                row[j] *= alpha[c];
        }
        /* u = S^T k */
        for (int j = 0; j < V; ++j)
            u[j] = 0.0;
        for (int c = 0; c < K; ++c) {
            const double kc = (double)kt[c];
            const double *row = S + (size_t)c * V;
            for (int j = 0; j < V; ++j)
                u[j] += row[j] * kc;
        }
        /* S <- S + beta k (v - u)^T */
        for (int j = 0; j < V; ++j)
            u[j] = b * ((double)vt[j] - u[j]);
        for (int c = 0; c < K; ++c) {
            const double kc = (double)kt[c];
            double *row = S + (size_t)c * V;
            for (int j = 0; j < V; ++j)
                row[j] += kc * u[j];
        }
        /* o = S^T q, read after the write */
        if (o) {
            double *ot = o + (long)t * o_stride;
            for (int j = 0; j < V; ++j)
                ot[j] = 0.0;
            for (int c = 0; c < K; ++c) {
                const double qc = (double)qt[c];
                const double *row = S + (size_t)c * V;
                for (int j = 0; j < V; ++j)
                    ot[j] += row[j] * qc;
            }
        }
    }
    free(alpha);
    free(u);
    return 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Number of threads an OpenMP parallel region would use now. */
int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Whole forward over [B, T, H]: every (b, h) slice is independent, one
 * OpenMP task per slice.  Returns 0, or -1 if any slice failed.
 */
int gdn_oracle_forward(int B, int T, int H, int K, int V, int channel_gate,
                       const float *q, const float *k, const float *v,
                       const float *g, const float *beta, const float *S0,
                       double *o, double *S_T, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0 || !S_T)
        return -1;
    set_threads(nthreads);
    const long nslice = (long)B * H;
    const long kv = (long)K * V;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long s = 0; s < nslice; ++s) {
        const long b = s / H, h = s % H;
        double *S = S_T + s * kv;
        if (S0) {
            for (long i = 0; i < kv; ++i)
                S[i] = (double)S0[s * kv + i];
        } else {
            memset(S, 0, sizeof(double) * (size_t)kv);
        }
        const long tok = (long)H;               /* token stride in rows */
        const long base = b * T * H + h;         /* row of token 0 */
        const long gk = channel_gate ? K : 1;
        failed |= gdn_oracle_slice(
            T, K, V, channel_gate,
            q + base * K, tok * K,
            k + base * K, tok * K,
            v + base * V, tok * V,
            g + base * gk, tok * gk,
            beta + base, tok,
            S, o ? o + base * V : NULL, tok * V) != 0;
    }
    return failed ? -1 : 0;
}

/*
 * Chained decode: steps tokens for each of N sequences and H heads, each token
 * one recurrent step of the state.  Inputs are [steps, N, H, ...]; S is
 * [N, H, K, V] doubles updated in place; o is [steps, N, H, V] or NULL.
 */
int gdn_oracle_decode(int steps, int N, int H, int K, int V, int channel_gate,
                      const float *q, const float *k, const float *v,
                      const float *g, const float *beta,
                      double *S, double *o, int nthreads)
{
    if (steps < 0 || N < 0 || H < 0 || K <= 0 || V <= 0 || !S)
        return -1;
    set_threads(nthreads);
    const long nslice = (long)N * H;
    const long kv = (long)K * V;
    const long gk = channel_gate ? K : 1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long s = 0; s < nslice; ++s) {
        failed |= gdn_oracle_slice(
            steps, K, V, channel_gate,
            q + s * K, nslice * K,
            k + s * K, nslice * K,
            v + s * V, nslice * V,
            g + s * gk, nslice * gk,
            beta + s, nslice,
            S + s * kv, o ? o + s * V : NULL, nslice * V) != 0;
    }
    return failed ? -1 : 0;
}
