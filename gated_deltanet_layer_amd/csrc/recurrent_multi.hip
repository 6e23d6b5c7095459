// recurrent_multi.hip -- M tokens per sequence from one state, in order: the
// verification step of speculative decoding (a few draft tokens scored from the
// state of the accepted prefix), between the one-token decode step and the
// chunkwise prefill.
//
// Every token is one step of the recurrence (Atomic-GDN2 model card, section
// 2.1), computed exactly as the one-token kernel (recurrent_step.hip) computes
// it:
//   u = S^T (alpha * k),  y = S^T (alpha * q),  delta = beta (v - u)
//   o = y + (k . q) delta,  S <- Diag(alpha) S + k delta^T
// The state block stays in registers for all M tokens: S is read once and the
// final state written once, whatever M is; optionally the state after every
// token is written too, so that the caller can roll back to any accepted
// prefix.
//
// Work split as in the one-token kernel: one 256-thread workgroup per (n, h,
// block of at most 64 value columns); thread t owns the float4 column group
// t % (VW/4) of rows t / (VW/4) + i * (256 / (VW/4)).  The per-token vectors
// (alpha k, alpha q, alpha, k) are double-buffered in LDS by token parity, so
// that a token's vectors can be written while the previous token's state update
// still reads its own.
//
// Occupancy: the kernel is bound by the state's round trip to HBM, and more
// workgroups in flight keep more of it moving.  It is compiled for five waves
// per SIMD (at most 96 VGPRs; d_k = d_v = 128 needs 92 then, with no spills,
// against 99 and four waves without the bound).
#include "gdn_common.h"

namespace gdn {

constexpr int RM_NTHR = 256;
constexpr int RM_NWAVE = RM_NTHR / 64;
constexpr int RM_VW = 64;             // value columns per workgroup (at most)

template <typename DT, int K, int V, bool CHANNEL>
__global__ __launch_bounds__(RM_NTHR) __attribute__((amdgpu_waves_per_eu(5))) void recurrent_multi_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *S0,
    DT *__restrict__ o, float *S_T, float *__restrict__ S_hist, int M, int H)
{
    constexpr int VW = V < RM_VW ? V : RM_VW;   // columns of this workgroup
    constexpr int NVW = V / VW;                 // workgroups per slice
    constexpr int TPR = VW / 4;       // threads per state row (float4 each)
    constexpr int RPP = RM_NTHR / TPR; // rows covered by one pass of the block
    constexpr int NP = K / RPP;       // passes
    static_assert(K % RPP == 0 && TPR <= 64 && 64 % TPR == 0, "unsupported K/V");

    __shared__ float s_ak[2][K];      // alpha * k
    __shared__ float s_aq[2][K];      // alpha * q
    __shared__ float s_al[2][K];      // alpha
    __shared__ float s_k[2][K];       // k
    __shared__ float s_qk[RM_NWAVE];
    __shared__ f32x4 s_red[RM_NWAVE][TPR][2];
    __shared__ f32x4 s_delta[TPR];

    const long slice = blockIdx.x / NVW;        // n H + h
    const long n = slice / H, h = slice % H;
    const int c0 = (blockIdx.x % NVW) * VW;     // first column of this workgroup
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col4 = tid % TPR;
    const int row0 = tid / TPR;

    // The state block, in registers for all M tokens (read once, non-temporal;
    // no S0 means zeros).
    f32x4 st[NP];
    if (S0) {
        const float *Sp = S0 + slice * (long)(K * V) + c0;
#pragma unroll
        for (int i = 0; i < NP; ++i)
            st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (row0 + i * RPP) * V + 4 * col4));
    } else {
#pragma unroll
        for (int i = 0; i < NP; ++i) st[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int j = 0; j < M; ++j) {
        const int b = j & 1;
        const long tok = (n * M + j) * H + h;   // row of token j in [N, M, H]
        float qk_part = 0.f;
        if (tid < K) {
            const float qc = to_f32(q[tok * K + tid]);
            const float kc = to_f32(k[tok * K + tid]);
            const float gc = CHANNEL ? g[tok * K + tid] : g[tok];
            const float a = __expf(gc);
            s_ak[b][tid] = a * kc;
            s_aq[b][tid] = a * qc;
            s_al[b][tid] = a;
            s_k[b][tid] = kc;
            qk_part = qc * kc;
        }
        qk_part = wave_sum(qk_part);
        if (lane == 0) s_qk[wave] = qk_part;
        __syncthreads();

        // Column partial sums over this thread's rows.
        f32x4 u = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int r = row0 + i * RPP;
            u += st[i] * s_ak[b][r];
            y += st[i] * s_aq[b][r];
        }
        // Reduce over the threads of a wave that share the column group.
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
            for (int w = 1; w < RM_NWAVE; ++w) {
                uu += s_red[w][tid][0];
                yy += s_red[w][tid][1];
                qk += s_qk[w];
            }
            const float bt = beta[tok];
            f32x4 d, oo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float ve = to_f32(v[tok * V + c0 + 4 * tid + e]);
                d[e] = bt * (ve - uu[e]);
                oo[e] = yy[e] + qk * d[e];
            }
            s_delta[tid] = d;
            if (o) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[tok * V + c0 + 4 * tid + e] = from_f32<DT>(oo[e]);
            }
        }
        __syncthreads();

        const f32x4 d = s_delta[col4];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int r = row0 + i * RPP;
            st[i] = st[i] * s_al[b][r] + d * s_k[b][r];
        }
        if (S_hist) {
            float *Hp = S_hist + tok * (long)(K * V) + c0;
#pragma unroll
            for (int i = 0; i < NP; ++i)
                __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4 *>(Hp + (row0 + i * RPP) * V + 4 * col4));
        }
    }

    if (S_T) {
        float *Tp = S_T + slice * (long)(K * V) + c0;
#pragma unroll
        for (int i = 0; i < NP; ++i)
            __builtin_nontemporal_store(st[i], reinterpret_cast<f32x4 *>(Tp + (row0 + i * RPP) * V + 4 * col4));
    }
}

template <typename DT, int K, int V, bool CH>
static hipError_t launch_multi(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *S0, void *o, float *S_T,
                               float *S_hist, long nslices, int M, int H, hipStream_t stream)
{
    constexpr int NVW = V / (V < RM_VW ? V : RM_VW);
    hipLaunchKernelGGL((recurrent_multi_kernel<DT, K, V, CH>), dim3((unsigned)(nslices * NVW)),
                       dim3(RM_NTHR), 0, stream, (const DT *)q, (const DT *)k, (const DT *)v, g,
                       beta, S0, (DT *)o, S_T, S_hist, M, H);
    return hipGetLastError();
}

template <typename DT, bool CH>
static hipError_t dispatch_multi(int K, int V, const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, const float *S0, void *o,
                                 float *S_T, float *S_hist, long nslices, int M, int H,
                                 hipStream_t st)
{
    if (K == 64 && V == 64)
        return launch_multi<DT, 64, 64, CH>(q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st);
    if (K == 64 && V == 128)
        return launch_multi<DT, 64, 128, CH>(q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st);
    if (K == 128 && V == 64)
        return launch_multi<DT, 128, 64, CH>(q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st);
    return launch_multi<DT, 128, 128, CH>(q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st);
}

// Host entry used by the C ABI after validation (nslices = N H > 0).
hipError_t recurrent_multi_launch(bool bf16, bool channel, int K, int V, const void *q,
                                  const void *k, const void *v, const float *g,
                                  const float *beta, const float *S0, void *o, float *S_T,
                                  float *S_hist, long nslices, int M, int H, hipStream_t st)
{
    if (bf16)
        return channel ? dispatch_multi<__bf16, true>(K, V, q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st)
                       : dispatch_multi<__bf16, false>(K, V, q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st);
    return channel ? dispatch_multi<float, true>(K, V, q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st)
                   : dispatch_multi<float, false>(K, V, q, k, v, g, beta, S0, o, S_T, S_hist, nslices, M, H, st);
}

} // namespace gdn
