// recurrent_step.hip -- fused recurrent (decode) step of the gated delta rule.
//
// One new token per (sequence n, head h).  With alpha = exp(g):
//   S' = (I - beta k k^T) Diag(alpha) S + beta k v^T,   o = S'^T q
// (Atomic-GDN2 model card, section 2.1).  Rewritten so that S is read once:
//   u     = S^T (alpha * k)          (what the memory returns for k)
//   y     = S^T (alpha * q)
//   delta = beta (v - u)
//   o     = y + (k . q) delta        since S'^T q = S^T(alpha*q) + delta (k^T q)
//   S'    = Diag(alpha) S + k delta^T
// Decoupled erase/write gates (the MindPattern page's split of beta into two
// gates; erase e in beta's place in the removal term, write gate w in the write
// term): S' = (I - e k k^T) Diag(alpha) S + w k v^T, so delta = w v - e u and the
// rest is unchanged.  wg == nullptr means w = beta.
// The step is HBM-bound: per slice it moves 2 * K * V * 4 bytes of state and a
// few hundred bytes of vectors; it uses plain fp32 VALU work and wave-level
// reductions, no matrix cores.
//
// Work split: columns of S never mix, so each (n, h) slice is split into blocks
// of at most 64 value columns, one 256-thread workgroup per block (twice the
// workgroups of one per slice, which keeps more of the state in flight).
// Thread t owns the float4 column group t % (VW/4) of rows t / (VW/4) +
// i * (256 / (VW/4)), so one wave-wide load covers whole 256-byte row pieces.
// The block stays in registers between the two reductions and the write-back,
// so S is read once and written once, in place.  A block belongs to exactly one
// workgroup, so the in-place update has no races.
#include "gdn_common.h"

namespace gdn {

constexpr int RS_NTHR = 256;
constexpr int RS_NWAVE = RS_NTHR / 64;
constexpr int RS_VW = 64;             // value columns per workgroup (at most)

template <typename DT, int K, int V, bool CHANNEL>
__global__ __launch_bounds__(RS_NTHR) void recurrent_step_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *__restrict__ wg, float *__restrict__ S, DT *__restrict__ o)
{
    constexpr int VW = V < RS_VW ? V : RS_VW;   // columns of this workgroup
    constexpr int NVW = V / VW;                 // workgroups per slice
    constexpr int TPR = VW / 4;       // threads per state row (float4 each)
    constexpr int RPP = RS_NTHR / TPR; // rows covered by one pass of the block
    constexpr int NP = K / RPP;       // passes
    static_assert(K % RPP == 0 && TPR <= 64 && 64 % TPR == 0, "unsupported K/V");

    __shared__ float s_ak[K];         // alpha * k
    __shared__ float s_aq[K];         // alpha * q
    __shared__ float s_al[K];         // alpha
    __shared__ float s_k[K];          // k
    __shared__ float s_qk[RS_NWAVE];
    __shared__ f32x4 s_red[RS_NWAVE][TPR][2];
    __shared__ f32x4 s_delta[TPR];

    const long slice = blockIdx.x / NVW;
    const int c0 = (blockIdx.x % NVW) * VW;     // first column of this workgroup
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col4 = tid % TPR;
    const int row0 = tid / TPR;

    // Issue the state loads first so they are in flight during the small loads.
    // The state streams through once per step, far larger than the caches, so
    // its loads and stores are marked non-temporal.
    float *Sp = S + slice * (long)(K * V) + c0;
    f32x4 st[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i)
        st[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sp + (row0 + i * RPP) * V + 4 * col4));

    float qk_part = 0.f;
    if (tid < K) {
        const float qc = to_f32(q[slice * K + tid]);
        const float kc = to_f32(k[slice * K + tid]);
        const float gc = CHANNEL ? g[slice * K + tid] : g[slice];
        const float a = __expf(gc);
        s_ak[tid] = a * kc;
        s_aq[tid] = a * qc;
        s_al[tid] = a;
        s_k[tid] = kc;
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
        u += st[i] * s_ak[r];
        y += st[i] * s_aq[r];
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
        for (int w = 1; w < RS_NWAVE; ++w) {
            uu += s_red[w][tid][0];
            yy += s_red[w][tid][1];
            qk += s_qk[w];
        }
        const float b = beta[slice];
        const float w = wg ? wg[slice] : 0.f;
        f32x4 d, oo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float ve = to_f32(v[slice * V + c0 + 4 * tid + e]);
            d[e] = wg ? w * ve - b * uu[e] : b * (ve - uu[e]);
            oo[e] = yy[e] + qk * d[e];
        }
        s_delta[tid] = d;
        if (o) {
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

template <typename DT, int K, int V, bool CH>
static hipError_t launch_step(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, const float *wg, float *S, void *o, long nslices,
                              hipStream_t stream)
{
    constexpr int NVW = V / (V < RS_VW ? V : RS_VW);
    hipLaunchKernelGGL((recurrent_step_kernel<DT, K, V, CH>), dim3((unsigned)(nslices * NVW)), dim3(RS_NTHR),
                       0, stream, (const DT *)q, (const DT *)k, (const DT *)v, g, beta, wg, S,
                       (DT *)o);
    return hipGetLastError();
}

template <typename DT, bool CH>
static hipError_t dispatch_kv(int K, int V, const void *q, const void *k, const void *v,
                              const float *g, const float *beta, const float *wg, float *S,
                              void *o, long nslices, hipStream_t st)
{
    if (K == 64 && V == 64) return launch_step<DT, 64, 64, CH>(q, k, v, g, beta, wg, S, o, nslices, st);
    if (K == 64 && V == 128) return launch_step<DT, 64, 128, CH>(q, k, v, g, beta, wg, S, o, nslices, st);
    if (K == 128 && V == 64) return launch_step<DT, 128, 64, CH>(q, k, v, g, beta, wg, S, o, nslices, st);
    return launch_step<DT, 128, 128, CH>(q, k, v, g, beta, wg, S, o, nslices, st);
}

// Host entry used by the C ABI after validation.  wg: the decoupled write gate,
// or nullptr (beta both erases and writes).
hipError_t recurrent_step_launch(bool bf16, bool channel, int K, int V, const void *q,
                                 const void *k, const void *v, const float *g,
                                 const float *beta, const float *wg, float *S, void *o,
                                 long nslices, hipStream_t st)
{
    if (bf16)
        return channel ? dispatch_kv<__bf16, true>(K, V, q, k, v, g, beta, wg, S, o, nslices, st)
                       : dispatch_kv<__bf16, false>(K, V, q, k, v, g, beta, wg, S, o, nslices, st);
    return channel ? dispatch_kv<float, true>(K, V, q, k, v, g, beta, wg, S, o, nslices, st)
                   : dispatch_kv<float, false>(K, V, q, k, v, g, beta, wg, S, o, nslices, st);
}

} // namespace gdn
