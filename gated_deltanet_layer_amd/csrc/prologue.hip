// prologue.hip -- the steps between the projections and the recurrence, and the
// decode step with those steps fused in.
//
// Per token (the raw q, k, v, g_raw, b_raw come from the layer's projections):
//   q, k, v  <- causal depthwise 4-tap convolution over time, per channel (the
//               kernel-4 convolution of the DeltaNet layers: "Hybrid layouts:
//               three DeltaNet, one attention", 01 Concept); tap j multiplies
//               token t - 3 + j; the three tokens before the sequence come from
//               a carried state (zeros if absent)
//            <- optional SiLU
//   q, k     <- divided by their L2 norm over the K channels of their head
//   g        <- -min(softplus(g_raw), cap)      (cap 5 on the Atomic-GDN2 card,
//   beta     <- sigmoid(b_raw)                   section 2.1)
// gdn_prologue runs these for a whole chunk-mode call in one launch (plus a tiny
// launch that writes the carried state out, so that it may be updated in place);
// gdn_recurrent_step_prologue runs them inside the one-token decode step, so
// that a decode token is one kernel from the raw projections to o and S'.
#include "gdn_common.h"
#include "prologue.h"
#include "prologue_ops.h"

namespace gdn {

constexpr int PR_NTHR = 256;

// 8 consecutive elements of a row as fp32 (16-byte loads).
template <typename DT> __device__ __forceinline__ void ld8(const DT *p, float (&x)[8]);
template <> __device__ __forceinline__ void ld8<float>(const float *p, float (&x)[8])
{
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = a[e];
        x[4 + e] = b[e];
    }
}
template <> __device__ __forceinline__ void ld8<__bf16>(const __bf16 *p, float (&x)[8])
{
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
}
// 8 consecutive elements of a row kept in their storage type until used.
template <typename DT> struct Raw8;
template <> struct Raw8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const f32x4 *>(p);
        b = *reinterpret_cast<const f32x4 *>(p + 4);
    }
    __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    }
};
template <> struct Raw8<__bf16> {
    bf16x8 a;
    __device__ __forceinline__ void load(const __bf16 *p) { a = __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p)); }
    __device__ __forceinline__ void get(float (&x)[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
    }
};
template <typename DT> __device__ __forceinline__ void st8(DT *p, const float (&x)[8]);
template <> __device__ __forceinline__ void st8<float>(float *p, const float (&x)[8])
{
    *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
template <> __device__ __forceinline__ void st8<__bf16>(__bf16 *p, const float (&x)[8])
{
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (__bf16)x[e];
    __builtin_nontemporal_store(a, reinterpret_cast<bf16x8 *>(p));
}

// Segments: q, k, v and the gates (blockIdx.y 1, 2, 3 and 0).  A thread owns 8 channels of
// one head and walks PR_TT consecutive tokens with the taps in registers and a
// sliding window of the last four raw rows, so each token costs one 16-byte
// load.  The K/8 threads of one head are consecutive lanes on the same tokens
// and reduce the squared norm with shuffles; consecutive heads follow, so a
// wave reads whole token rows.
constexpr int PR_TT = 16;

constexpr unsigned ilog2c(unsigned x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

template <typename DT, int W, bool NORM, bool SILU>
__device__ __forceinline__ void conv_run(const DT *x, const DT *cs, const float *w, DT *y, long b,
                                         int t0, int T, int D, int c)
{
    f32x4 wt[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) wt[e] = *reinterpret_cast<const f32x4 *>(w + (long)(c + e) * 4);
    float win[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int tt = t0 - 3 + j;
        if (tt >= 0) {
            ld8(x + (b * T + tt) * (long)D + c, win[j]);
        } else if (cs) {
            ld8(cs + (b * 3 + (tt + 3)) * (long)D + c, win[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
        }
    }
    auto token = [&](int t, const float (&xt)[8]) {
        float o[8];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = pr_conv4(wt[e], win[0][e], win[1][e], win[2][e], xt[e]);
            o[e] = SILU ? pr_silu(v) : v;
            ss = fmaf(o[e], o[e], ss);
        }
        if (NORM) {
#pragma unroll
            for (int off = 1; off < W; off <<= 1) ss += __shfl_xor(ss, off, W);
            const float rn = pr_rnorm(ss);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= rn;
        }
        st8(y + (b * T + t) * (long)D + c, o);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            win[0][e] = win[1][e];
            win[1][e] = win[2][e];
            win[2][e] = xt[e];
        }
    };
    if (t0 + PR_TT <= T) {
        // a whole block of tokens (the same for every lane of a head): all of
        // its loads in flight before the first token is computed
        Raw8<DT> xs[PR_TT];
#pragma unroll
        for (int i = 0; i < PR_TT; ++i) xs[i].load(x + (b * T + t0 + i) * (long)D + c);
#pragma unroll
        for (int i = 0; i < PR_TT; ++i) {
            float xt[8];
            xs[i].get(xt);
            token(t0 + i, xt);
        }
    } else {
        for (int t = t0; t < T; ++t) {
            float xt[8];
            ld8(x + (b * T + t) * (long)D + c, xt);
            token(t, xt);
        }
    }
}

template <typename DT, int K, int V, bool CH, bool SILU>
__global__ __launch_bounds__(PR_NTHR) void prologue_kernel(PrArgs a)
{
    // The entry point keeps 16 work items per token below 2^32, so the index
    // arithmetic is 32-bit (a 64-bit division by a run-time value costs a long
    // instruction sequence per thread).
    const unsigned idx = blockIdx.x * PR_NTHR + threadIdx.x;
    // the small gates segment first in dispatch order, so that it runs beside
    // the convolutions instead of after them
    const int seg = blockIdx.y == 0 ? 3 : blockIdx.y - 1;
    const unsigned NTB = (a.T + PR_TT - 1) / PR_TT, Hu = a.H;
    const unsigned long long rows = (unsigned long long)a.B * NTB * Hu;   // (b, token block, h)
    if (seg <= 2) {
        const int E = seg == 2 ? V : K;
        const unsigned lg = seg == 2 ? ilog2c(V / 8) : ilog2c(K / 8);   // lanes per (token block, head): 2^lg
        if (idx >= (rows << lg)) return;                                // whole groups of lanes
        const unsigned r = idx >> lg;
        const int h = (int)(r % Hu);
        const unsigned btb = r / Hu;
        const int tb = (int)(btb % NTB);
        const long b = btb / NTB;
        const int D = a.H * E, c = h * E + (int)(idx & ((1u << lg) - 1)) * 8;
        if (seg == 0)
            conv_run<DT, K / 8, true, SILU>((const DT *)a.q_raw, (const DT *)a.cs_q, a.w_q,
                                            (DT *)a.q, b, tb * PR_TT, a.T, D, c);
        else if (seg == 1)
            conv_run<DT, K / 8, true, SILU>((const DT *)a.k_raw, (const DT *)a.cs_k, a.w_k,
                                            (DT *)a.k, b, tb * PR_TT, a.T, D, c);
        else
            conv_run<DT, V / 8, false, SILU>((const DT *)a.v_raw, (const DT *)a.cs_v, a.w_v,
                                             (DT *)a.v, b, tb * PR_TT, a.T, D, c);
    } else {
        constexpr unsigned G = CH ? K / 4 : 1;
        if (idx >= rows * G) return;
        const unsigned r = idx / G;
        const int h = (int)(r % Hu);
        const unsigned btb = r / Hu;
        const int tb = (int)(btb % NTB);
        const long b = btb / NTB;
        const int x0 = (int)(idx % G) * 4;
        const int t0 = tb * PR_TT, nt = min(PR_TT, a.T - t0);
        const long row0 = (b * a.T + t0) * a.H + h;   // token t0 + i: row0 + i H
        // every load of the block in flight before the first is used (rows past
        // the end re-read the last one and are not stored)
        f32x4 gr[PR_TT];
        float br[PR_TT];
#pragma unroll
        for (int i = 0; i < PR_TT; ++i) {
            const long row = row0 + (long)min(i, nt - 1) * a.H;
            if (CH) gr[i] = *reinterpret_cast<const f32x4 *>(a.g_raw + row * K + x0);
            else gr[i][0] = a.g_raw[row];
            br[i] = (!CH || x0 == 0) ? a.b_raw[row] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < PR_TT; ++i) {
            if (i < nt) {
                const long row = row0 + (long)i * a.H;
                if (CH) {
                    f32x4 gv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) gv[e] = pr_gate(gr[i][e], a.cap);
                    *reinterpret_cast<f32x4 *>(a.g + row * K + x0) = gv;
                    if (x0 == 0) a.beta[row] = pr_sigmoid(br[i]);
                } else {
                    a.g[row] = pr_gate(gr[i][0], a.cap);
                    a.beta[row] = pr_sigmoid(br[i]);
                }
            }
        }
    }
}

// The carried states after the sequence: the last three raw tokens (older ones
// from the incoming state when T < 3).  One thread reads all three rows of its
// 8 channels before writing any, so the output may be the incoming state.
template <typename DT>
__device__ __forceinline__ void state_out8(const DT *x, const DT *cs, DT *out, long b, int T,
                                           int D, int c)
{
    float r[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int tt = T - 3 + j;
        if (tt >= 0) {
            ld8(x + (b * T + tt) * (long)D + c, r[j]);
        } else if (cs) {
            ld8(cs + (b * 3 + (tt + 3)) * (long)D + c, r[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) r[j][e] = 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) st8(out + (b * 3 + j) * (long)D + c, r[j]);
}

template <typename DT, int K, int V>
__global__ __launch_bounds__(PR_NTHR) void prologue_state_kernel(PrArgs a)
{
    const long idx = (long)blockIdx.x * PR_NTHR + threadIdx.x;
    const int seg = blockIdx.y;
    const int D = a.H * (seg == 2 ? V : K);
    if (idx >= (long)a.B * (D / 8)) return;
    const long b = idx / (D / 8);
    const int c = (int)(idx % (D / 8)) * 8;
    const DT *x = (const DT *)(seg == 0 ? a.q_raw : seg == 1 ? a.k_raw : a.v_raw);
    const DT *cs = (const DT *)(seg == 0 ? a.cs_q : seg == 1 ? a.cs_k : a.cs_v);
    DT *out = (DT *)(seg == 0 ? a.cs_q_out : seg == 1 ? a.cs_k_out : a.cs_v_out);
    if (out) state_out8(x, cs, out, b, a.T, D, c);
}

template <typename DT, int K, int V, bool CH, bool SILU>
static hipError_t launch_prologue(const PrArgs &a, hipStream_t st)
{
    const long rows = (long)a.B * ((a.T + PR_TT - 1) / PR_TT) * a.H;
    long nthr = rows * (K / 8);
    nthr = nthr > rows * (V / 8) ? nthr : rows * (V / 8);
    nthr = nthr > rows * (CH ? K / 4 : 1) ? nthr : rows * (CH ? K / 4 : 1);
    if (rows > 0)
        hipLaunchKernelGGL((prologue_kernel<DT, K, V, CH, SILU>),
                           dim3((unsigned)((nthr + PR_NTHR - 1) / PR_NTHR), 4), dim3(PR_NTHR), 0, st, a);
    if (a.cs_q_out || a.cs_k_out || a.cs_v_out) {
        const long ns = (long)a.B * a.H * ((K > V ? K : V) / 8);
        hipLaunchKernelGGL((prologue_state_kernel<DT, K, V>),
                           dim3((unsigned)((ns + PR_NTHR - 1) / PR_NTHR), 3), dim3(PR_NTHR), 0, st, a);
    }
    return hipGetLastError();
}

template <typename DT, int K, int V>
static hipError_t dispatch_prologue_act(bool ch, bool silu, const PrArgs &a, hipStream_t st)
{
    if (ch) return silu ? launch_prologue<DT, K, V, true, true>(a, st) : launch_prologue<DT, K, V, true, false>(a, st);
    return silu ? launch_prologue<DT, K, V, false, true>(a, st) : launch_prologue<DT, K, V, false, false>(a, st);
}

template <typename DT>
static hipError_t dispatch_prologue(int K, int V, bool ch, bool silu, const PrArgs &a, hipStream_t st)
{
    if (K == 64 && V == 64) return dispatch_prologue_act<DT, 64, 64>(ch, silu, a, st);
    if (K == 64 && V == 128) return dispatch_prologue_act<DT, 64, 128>(ch, silu, a, st);
    if (K == 128 && V == 64) return dispatch_prologue_act<DT, 128, 64>(ch, silu, a, st);
    return dispatch_prologue_act<DT, 128, 128>(ch, silu, a, st);
}

hipError_t prologue_launch(bool bf16, bool channel, bool silu, int K, int V, const PrArgs &a,
                           hipStream_t st)
{
    return bf16 ? dispatch_prologue<__bf16>(K, V, channel, silu, a, st)
                : dispatch_prologue<float>(K, V, channel, silu, a, st);
}

// ---------------------------------------------------------------- fused decode
// The one-token recurrence of recurrent_step.hip (one 256-thread workgroup per
// (n, h, block of at most 64 value columns); S read once, written once, in
// place), preceded by the prologue of that token.  The q and k of a slice are
// computed by every value block of it (they need them all); the carried q/k
// state is written by the first value block only, the v state by each block for
// its columns.  The state output therefore must not be the input.
constexpr int RP_VW = 64;

template <typename DT, int K, int V, bool CH, bool SILU>
__global__ __launch_bounds__(PR_NTHR) void recurrent_step_prologue_kernel(RpArgs a)
{
    constexpr int NW = PR_NTHR / 64;
    constexpr int VW = V < RP_VW ? V : RP_VW;
    constexpr int NVW = V / VW;
    constexpr int TPR = VW / 4;
    constexpr int RPP = PR_NTHR / TPR;
    constexpr int NP = K / RPP;
    static_assert(K % RPP == 0 && TPR <= 64 && 64 % TPR == 0 && K <= PR_NTHR, "unsupported K/V");

    __shared__ float s_ak[K], s_aq[K], s_al[K], s_k[K], s_v[VW];
    __shared__ float s_ss[2][NW], s_qk[NW];
    __shared__ f32x4 s_red[NW][TPR][2];
    __shared__ f32x4 s_delta[TPR];

    const long slice = blockIdx.x / NVW;          // n H + h
    const int vb = blockIdx.x % NVW, c0 = vb * VW;
    const long n = slice / a.H;
    const int h = (int)(slice % a.H);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col4 = tid % TPR, row0 = tid / TPR;
    const int DK = a.H * K, DV = a.H * V;

    float *Sp = a.S + slice * (long)(K * V) + c0;
    f32x4 st[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i)
        st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (row0 + i * RPP) * V + 4 * col4));

    // the prologue: q, k by channel (tid < K), v by column of this block (tid < VW)
    const DT *qr = (const DT *)a.q_raw, *kr = (const DT *)a.k_raw, *vr = (const DT *)a.v_raw;
    const DT *csq = (const DT *)a.cs_q, *csk = (const DT *)a.cs_k, *csv = (const DT *)a.cs_v;
    float yq = 0.f, yk = 0.f;
    if (tid < K) {
        const int c = h * K + tid;
        float xq[4], xk[4];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            xq[j] = csq ? to_f32(csq[(n * 3 + j) * DK + c]) : 0.f;
            xk[j] = csk ? to_f32(csk[(n * 3 + j) * DK + c]) : 0.f;
        }
        xq[3] = to_f32(qr[slice * K + tid]);
        xk[3] = to_f32(kr[slice * K + tid]);
        const f32x4 wq = *reinterpret_cast<const f32x4 *>(a.w_q + (long)c * 4);
        const f32x4 wk = *reinterpret_cast<const f32x4 *>(a.w_k + (long)c * 4);
        yq = fmaf(wq[3], xq[3], fmaf(wq[2], xq[2], fmaf(wq[1], xq[1], wq[0] * xq[0])));
        yk = fmaf(wk[3], xk[3], fmaf(wk[2], xk[2], fmaf(wk[1], xk[1], wk[0] * xk[0])));
        if (SILU) {
            yq = pr_silu(yq);
            yk = pr_silu(yk);
        }
        if (vb == 0) {
            DT *oq = (DT *)a.cs_q_out, *ok = (DT *)a.cs_k_out;
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                if (oq) oq[(n * 3 + j) * DK + c] = from_f32<DT>(xq[j + 1]);
                if (ok) ok[(n * 3 + j) * DK + c] = from_f32<DT>(xk[j + 1]);
            }
        }
    }
    if (tid < VW) {
        const int c = h * V + c0 + tid;
        float xv[4];
#pragma unroll
        for (int j = 0; j < 3; ++j) xv[j] = csv ? to_f32(csv[(n * 3 + j) * DV + c]) : 0.f;
        xv[3] = to_f32(vr[slice * V + c0 + tid]);
        const f32x4 wv = *reinterpret_cast<const f32x4 *>(a.w_v + (long)c * 4);
        float yv = fmaf(wv[3], xv[3], fmaf(wv[2], xv[2], fmaf(wv[1], xv[1], wv[0] * xv[0])));
        s_v[tid] = SILU ? pr_silu(yv) : yv;
        DT *ov = (DT *)a.cs_v_out;
        if (ov) {
#pragma unroll
            for (int j = 0; j < 3; ++j) ov[(n * 3 + j) * DV + c] = from_f32<DT>(xv[j + 1]);
        }
    }
    {
        const float sq = wave_sum(yq * yq), sk = wave_sum(yk * yk);
        if (lane == 0) {
            s_ss[0][wave] = sq;
            s_ss[1][wave] = sk;
        }
    }
    __syncthreads();
    float qk_part = 0.f;
    if (tid < K) {
        float nq = 0.f, nk = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            nq += s_ss[0][w];
            nk += s_ss[1][w];
        }
        const float qc = yq * pr_rnorm(nq), kc = yk * pr_rnorm(nk);
        const float gc = pr_gate(CH ? a.g_raw[slice * K + tid] : a.g_raw[slice], a.cap);
        const float al = __expf(gc);
        s_ak[tid] = al * kc;
        s_aq[tid] = al * qc;
        s_al[tid] = al;
        s_k[tid] = kc;
        qk_part = qc * kc;
    }
    qk_part = wave_sum(qk_part);
    if (lane == 0) s_qk[wave] = qk_part;
    __syncthreads();

    // the recurrence, as in recurrent_step.hip
    f32x4 u = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int r = row0 + i * RPP;
        u += st[i] * s_ak[r];
        y += st[i] * s_aq[r];
    }
#pragma unroll
    for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] += __shfl_xor(u[e], off, 64);
            y[e] += __shfl_xor(y[e], off, 64);
        }
    }
    if (lane < TPR) {
        s_red[wave][lane][0] = u;
        s_red[wave][lane][1] = y;
    }
    __syncthreads();
    if (tid < TPR) {
        f32x4 uu = s_red[0][tid][0], yy = s_red[0][tid][1];
        float qk = s_qk[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            uu += s_red[w][tid][0];
            yy += s_red[w][tid][1];
            qk += s_qk[w];
        }
        const float bt = pr_sigmoid(a.b_raw[slice]);
        f32x4 d, oo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            d[e] = bt * (s_v[4 * tid + e] - uu[e]);
            oo[e] = yy[e] + qk * d[e];
        }
        s_delta[tid] = d;
        if (a.o) {
            DT *o = (DT *)a.o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[slice * V + c0 + 4 * tid + e] = from_f32<DT>(oo[e]);
        }
    }
    __syncthreads();
    const f32x4 d = s_delta[col4];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int r = row0 + i * RPP;
        const f32x4 nv = st[i] * s_al[r] + d * s_k[r];
        __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(Sp + r * V + 4 * col4));
    }
}

template <typename DT, int K, int V, bool CH, bool SILU>
static hipError_t launch_step_prologue(const RpArgs &a, long nslices, hipStream_t st)
{
    constexpr int NVW = V / (V < RP_VW ? V : RP_VW);
    hipLaunchKernelGGL((recurrent_step_prologue_kernel<DT, K, V, CH, SILU>),
                       dim3((unsigned)(nslices * NVW)), dim3(PR_NTHR), 0, st, a);
    return hipGetLastError();
}

template <typename DT, int K, int V>
static hipError_t dispatch_step_act(bool ch, bool silu, const RpArgs &a, long ns, hipStream_t st)
{
    if (ch) return silu ? launch_step_prologue<DT, K, V, true, true>(a, ns, st)
                        : launch_step_prologue<DT, K, V, true, false>(a, ns, st);
    return silu ? launch_step_prologue<DT, K, V, false, true>(a, ns, st)
                : launch_step_prologue<DT, K, V, false, false>(a, ns, st);
}

template <typename DT>
static hipError_t dispatch_step_prologue(int K, int V, bool ch, bool silu, const RpArgs &a, long ns,
                                         hipStream_t st)
{
    if (K == 64 && V == 64) return dispatch_step_act<DT, 64, 64>(ch, silu, a, ns, st);
    if (K == 64 && V == 128) return dispatch_step_act<DT, 64, 128>(ch, silu, a, ns, st);
    if (K == 128 && V == 64) return dispatch_step_act<DT, 128, 64>(ch, silu, a, ns, st);
    return dispatch_step_act<DT, 128, 128>(ch, silu, a, ns, st);
}

hipError_t step_prologue_launch(bool bf16, bool channel, bool silu, int K, int V, const RpArgs &a,
                                long nslices, hipStream_t st)
{
    return bf16 ? dispatch_step_prologue<__bf16>(K, V, channel, silu, a, nslices, st)
                : dispatch_step_prologue<float>(K, V, channel, silu, a, nslices, st);
}

} // namespace gdn
