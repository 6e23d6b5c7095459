// chunk_bwd.hip -- chunkwise backward of the gated delta rule (fp32 arithmetic).
//
// Gradients of a loss through the recurrence of the Atomic-GDN2 model card,
// section 2.1 (S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
// o_t = S_t^T q_t, alpha_t = exp(g_t)), given dL/do and dL/dS_T; the same card
// times its kernel forward and backward together (section 5.1).  Inputs are the
// forward's inputs; nothing from the forward pass is kept, the states are
// recomputed.
//
// Chunk algebra (C = 64 tokens, one (batch, head) slice, chunk entered with
// state S; gamma = in-chunk cumulative log-decay per key channel, gn its last
// row; rows past the end of the sequence are zero with g = 0):
//   Kp = k e^{gamma},  Qp = q e^{gamma},  Km = k e^{gn - gamma}
//   G_ts = sum_c k_tc k_sc e^{gamma_tc - gamma_sc} (s < t),  P_ts likewise with q_t (s <= t)
//   T = (I + diag(beta) G)^{-1},  Delta = T diag(beta) (V - Kp S)
//   O = Qp S + P Delta,  S' = Diag(e^{gn}) S + Km^T Delta
// Reverse mode of those lines, with dS' = dL/dS' carried backwards over chunks:
//   dDelta = Km dS' + P^T dO,   Y = T^T dDelta
//   dS     = Diag(e^{gn}) dS' + Qp^T dO - Kp^T diag(beta) Y
//   dv = beta Y,  dbeta += rowsum(V * Y),  dT = dDelta (beta V)^T - dDelta S^T (beta Kp)^T
//   dQp = dO S^T,  dKm = Delta dS'^T,  Z = -T^T dDelta S^T = dL/d(beta Kp),  dP = dO Delta^T
//   dA = -T^T dT T^T (strictly lower),  dG = diag(beta) dA,  dbeta += rowsum(dA * G)
// then the chain rule through G, P, Kp, Qp, Km to dq, dk and d gamma, and
// dg = reverse cumulative sum of d gamma over the chunk (plus the gn terms on
// its last row); a scalar gate sums dg over the key channels.
//
// Kernels, in stream order (each launch covers every slice):
//   1 prep     one workgroup per chunk:   gamma, G, P, T
//   2 states   one per value block:       walks the chunks forward; the state
//                                         entering each chunk and Delta
//   3 dstates  one per value block:       walks them backward; dL/dS' of each
//                                         chunk, dDelta, and dS0
//   4 vgrad    one per chunk:             every product that sums over the
//                                         value dimension; dv
//   5 kgrad    one per chunk:             the rest; dq, dk, dg, dbeta
// The state recursions split by value column (column j of S and of dS depends
// only on column j), which is what lets 2 and 3 run one workgroup per block of
// value columns.  Intermediates live in a caller-provided fp32 workspace.
//
// Products are LDS-tiled fp32 FMAs: each thread owns a small output tile whose
// rows and columns are interleaved across the workgroup, so that the operand
// reads of a wave hit consecutive or odd-strided LDS addresses.
#include "gdn_common.h"
#include "chunk_bwd.h"

namespace gdn {

constexpr int BW_C = 64;
constexpr int BW_NTHR = 256;

// acc[i][j] += sum_{x < KD} A[(mt + i*MS) AM + x AK] * B[x BK + (nt + j*NS) BN]
// with MS = M / TM and NS = N / TN: the thread's tile is rows mt + i*MS and
// columns nt + j*NS of an M x N output.
template <int M, int N, int TM, int TN, int KD, int AM, int AK, int BK, int BN>
__device__ __forceinline__ void mm_acc(float (&acc)[TM][TN], const float *A, const float *B,
                                       int mt, int nt)
{
    constexpr int MS = M / TM, NS = N / TN;
#pragma unroll 4
    for (int x = 0; x < KD; ++x) {
        float a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = A[(mt + i * MS) * AM + x * AK];
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = B[x * BK + (nt + j * NS) * BN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
}

// One tile per thread: (M/TM) x (N/TN) == 256.
template <int M, int N, int TM, int TN> struct Tile {
    static_assert(M % TM == 0 && N % TN == 0 && (M / TM) * (N / TN) == BW_NTHR, "tile map");
    static constexpr int MS = M / TM, NS = N / TN;
    int mt, nt;
    __device__ __forceinline__ Tile() : mt(threadIdx.x / NS), nt(threadIdx.x % NS) {}
    __device__ __forceinline__ int row(int i) const { return mt + i * MS; }
    __device__ __forceinline__ int col(int j) const { return nt + j * NS; }
};

// Row of token t of slice sl in the [B, T, H] token layout.
__device__ __forceinline__ long tok_row(const BwArgs &a, int sl, int t)
{
    const long b = sl / a.H, h = sl % a.H;
    return (b * a.T + t) * a.H + h;
}

// ---------------------------------------------------------------- 1 prep
template <typename DT, int K, bool CH>
__global__ __launch_bounds__(BW_NTHR) void bwd_prep_kernel(BwArgs a)
{
    constexpr int C = BW_C, KP = K + 1, CP = C + 1;
    extern __shared__ __attribute__((aligned(256))) float sm[];
    float *sk = sm, *sq = sk + C * KP, *sg = sq + C * KP, *sA = sg + C * KP, *sT = sA + C * CP;
    float *sb = sT + C * CP;
    const int tid = threadIdx.x;
    const int c = blockIdx.x % a.NC, sl = blockIdx.x / a.NC;
    const int t0 = c * C, n = min(C, a.T - t0);
    const long ci = (long)sl * a.NC + c;
    const DT *q = (const DT *)a.q, *k = (const DT *)a.k;

    for (int idx = tid; idx < C * K; idx += BW_NTHR) {
        const int t = idx / K, x = idx % K;
        float kv = 0.f, qv = 0.f, gv = 0.f;
        if (t < n) {
            const long r = tok_row(a, sl, t0 + t);
            kv = to_f32(k[r * K + x]);
            qv = to_f32(q[r * K + x]);
            gv = CH ? a.g[r * K + x] : a.g[r];
        }
        sk[t * KP + x] = kv;
        sq[t * KP + x] = qv;
        sg[t * KP + x] = gv;
    }
    if (tid < C) sb[tid] = tid < n ? a.beta[tok_row(a, sl, t0 + tid)] : 0.f;
    __syncthreads();
    if (tid < K) {   // gamma: running sum over the chunk, one channel per thread
        float acc = 0.f;
        for (int t = 0; t < C; ++t) {
            acc += sg[t * KP + tid];
            sg[t * KP + tid] = acc;
        }
    }
    __syncthreads();
    float *gam = a.ws.gam + ci * (C * K);
    for (int idx = tid; idx < C * K; idx += BW_NTHR) gam[idx] = sg[(idx / K) * KP + idx % K];

    // G and P over the pairs s <= t (2080 of them), one pair per thread at a time
    float *Gm = a.ws.Gm + ci * (C * C), *Pm = a.ws.Pm + ci * (C * C);
    for (int p = tid; p < C * (C + 1) / 2; p += BW_NTHR) {
        int t = (int)((sqrtf(8.f * (float)p + 1.f) - 1.f) * 0.5f);
        while (t * (t + 1) / 2 > p) --t;
        while ((t + 1) * (t + 2) / 2 <= p) ++t;
        const int s = p - t * (t + 1) / 2;
        float gk = 0.f, pq = 0.f;
        for (int x = 0; x < K; ++x) {
            const float ks = sk[s * KP + x] * __expf(sg[t * KP + x] - sg[s * KP + x]);
            gk = fmaf(sk[t * KP + x], ks, gk);
            pq = fmaf(sq[t * KP + x], ks, pq);
        }
        const float gts = s < t ? gk : 0.f;
        Gm[t * C + s] = gts;
        Pm[t * C + s] = pq;
        sA[t * CP + s] = sb[t] * gts;
    }
    for (int idx = tid; idx < C * C; idx += BW_NTHR) {
        const int t = idx / C, s = idx % C;
        if (s > t) {
            Gm[idx] = 0.f;
            Pm[idx] = 0.f;
            sA[t * CP + s] = 0.f;
        }
    }
    __syncthreads();
    // T = (I + A)^{-1} by forward substitution, one column per thread
    if (tid < C) {
        const int j = tid;
        for (int i = 0; i < C; ++i) {
            float acc = i == j ? 1.f : 0.f;
            for (int s = 0; s < i; ++s) acc = fmaf(-sA[i * CP + s], sT[s * CP + j], acc);
            sT[i * CP + j] = acc;
        }
    }
    __syncthreads();
    float *Tm = a.ws.Tm + ci * (C * C);
    for (int idx = tid; idx < C * C; idx += BW_NTHR) Tm[idx] = sT[(idx / C) * CP + idx % C];
}

// ---------------------------------------------------------------- 2 states
template <typename DT, int K, int V, bool CH>
__global__ __launch_bounds__(BW_NTHR) void bwd_states_kernel(BwArgs a)
{
    constexpr int C = BW_C, VB = bw_vb(K), KP = K + 1, CP = C + 1, VP = VB + 1, NVB = V / VB;
    extern __shared__ __attribute__((aligned(256))) float sm[];
    float *sKp = sm, *sKm = sKp + C * KP, *sT = sKm + C * KP, *sS = sT + C * CP;
    float *sR = sS + K * VP, *sD = sR + C * VP, *sb = sD + C * VP, *sgn = sb + C;
    const int tid = threadIdx.x;
    const int vb = blockIdx.x % NVB, sl = blockIdx.x / NVB, v0 = vb * VB;
    const DT *k = (const DT *)a.k, *v = (const DT *)a.v;

    for (int idx = tid; idx < K * VB; idx += BW_NTHR) {
        const int x = idx / VB, y = idx % VB;
        sS[x * VP + y] = a.S0 ? a.S0[((long)sl * K + x) * V + v0 + y] : 0.f;
    }
    for (int c = 0; c < a.NC; ++c) {
        const int t0 = c * C, n = min(C, a.T - t0);
        const long ci = (long)sl * a.NC + c;
        const float *gam = a.ws.gam + ci * (C * K);
        __syncthreads();   // the previous chunk's readers are done
        for (int idx = tid; idx < C * K; idx += BW_NTHR) {
            const int t = idx / K, x = idx % K;
            const float kv = t < n ? to_f32(k[tok_row(a, sl, t0 + t) * K + x]) : 0.f;
            const float gm = gam[idx], gn = gam[(C - 1) * K + x];
            sKp[t * KP + x] = kv * __expf(gm);
            sKm[t * KP + x] = kv * __expf(gn - gm);
        }
        if (tid < K) sgn[tid] = __expf(gam[(C - 1) * K + tid]);
        const float *Tm = a.ws.Tm + ci * (C * C);
        for (int idx = tid; idx < C * C; idx += BW_NTHR) sT[(idx / C) * CP + idx % C] = Tm[idx];
        for (int idx = tid; idx < C * VB; idx += BW_NTHR) {
            const int t = idx / VB, y = idx % VB;
            sR[t * VP + y] = t < n ? to_f32(v[tok_row(a, sl, t0 + t) * V + v0 + y]) : 0.f;
        }
        if (tid < C) sb[tid] = tid < n ? a.beta[tok_row(a, sl, t0 + tid)] : 0.f;
        float *hS = a.ws.hS + ci * (K * V);
        for (int idx = tid; idx < K * VB; idx += BW_NTHR) {
            const int x = idx / VB, y = idx % VB;
            hS[x * V + v0 + y] = sS[x * VP + y];
        }
        __syncthreads();
        {   // R = beta (V - Kp S), in place over the v tile
            using TL = Tile<C, VB, 4, VB / 16>;
            const TL tl;
            float acc[4][VB / 16] = {};
            mm_acc<C, VB, 4, VB / 16, K, KP, 1, VP, 1>(acc, sKp, sS, tl.mt, tl.nt);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < VB / 16; ++j) {
                    const int t = tl.row(i), y = tl.col(j);
                    sR[t * VP + y] = sb[t] * (sR[t * VP + y] - acc[i][j]);
                }
        }
        __syncthreads();
        {   // Delta = T R
            using TL = Tile<C, VB, 4, VB / 16>;
            const TL tl;
            float acc[4][VB / 16] = {};
            mm_acc<C, VB, 4, VB / 16, C, CP, 1, VP, 1>(acc, sT, sR, tl.mt, tl.nt);
            float *Dl = a.ws.Dl + ci * (C * V);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < VB / 16; ++j) {
                    const int t = tl.row(i), y = tl.col(j);
                    sD[t * VP + y] = acc[i][j];
                    Dl[t * V + v0 + y] = acc[i][j];
                }
        }
        __syncthreads();
        {   // S = Diag(e^{gn}) S + Km^T Delta
            using TL = Tile<K, VB, K / 16, VB / 16>;
            const TL tl;
            float acc[K / 16][VB / 16] = {};
            mm_acc<K, VB, K / 16, VB / 16, C, 1, KP, VP, 1>(acc, sKm, sD, tl.mt, tl.nt);
#pragma unroll
            for (int i = 0; i < K / 16; ++i)
#pragma unroll
                for (int j = 0; j < VB / 16; ++j) {
                    const int x = tl.row(i), y = tl.col(j);
                    sS[x * VP + y] = sgn[x] * sS[x * VP + y] + acc[i][j];
                }
        }
    }
}

// ---------------------------------------------------------------- 3 dstates
template <typename DT, int K, int V, bool CH>
__global__ __launch_bounds__(BW_NTHR) void bwd_dstates_kernel(BwArgs a)
{
    constexpr int C = BW_C, VB = bw_vb(K), KP = K + 1, CP = C + 1, VP = VB + 1, NVB = V / VB;
    extern __shared__ __attribute__((aligned(256))) float sm[];
    float *sQK = sm;                 // rows 0..C-1: Qp, rows C..2C-1: Kp
    float *sKm = sQK + 2 * C * KP, *sP = sKm + C * KP, *sT = sP + C * CP, *sdS = sT + C * CP;
    float *sOY = sdS + K * VP;       // rows 0..C-1: dO, rows C..2C-1: -beta Y
    float *sdD = sOY + 2 * C * VP, *sb = sdD + C * VP, *sgn = sb + C;
    const int tid = threadIdx.x;
    const int vb = blockIdx.x % NVB, sl = blockIdx.x / NVB, v0 = vb * VB;
    const DT *q = (const DT *)a.q, *k = (const DT *)a.k, *dO = (const DT *)a.d_o;

    for (int idx = tid; idx < K * VB; idx += BW_NTHR) {
        const int x = idx / VB, y = idx % VB;
        sdS[x * VP + y] = a.dS_T ? a.dS_T[((long)sl * K + x) * V + v0 + y] : 0.f;
    }
    for (int c = a.NC - 1; c >= 0; --c) {
        const int t0 = c * C, n = min(C, a.T - t0);
        const long ci = (long)sl * a.NC + c;
        const float *gam = a.ws.gam + ci * (C * K);
        __syncthreads();
        for (int idx = tid; idx < C * K; idx += BW_NTHR) {
            const int t = idx / K, x = idx % K;
            float kv = 0.f, qv = 0.f;
            if (t < n) {
                const long r = tok_row(a, sl, t0 + t);
                kv = to_f32(k[r * K + x]);
                qv = to_f32(q[r * K + x]);
            }
            const float gm = gam[idx], gn = gam[(C - 1) * K + x], e = __expf(gm);
            sQK[t * KP + x] = qv * e;
            sQK[(C + t) * KP + x] = kv * e;
            sKm[t * KP + x] = kv * __expf(gn - gm);
        }
        if (tid < K) sgn[tid] = __expf(gam[(C - 1) * K + tid]);
        const float *Pm = a.ws.Pm + ci * (C * C), *Tm = a.ws.Tm + ci * (C * C);
        for (int idx = tid; idx < C * C; idx += BW_NTHR) {
            const int t = idx / C, s = idx % C;
            sP[t * CP + s] = Pm[idx];
            sT[t * CP + s] = Tm[idx];
        }
        for (int idx = tid; idx < C * VB; idx += BW_NTHR) {
            const int t = idx / VB, y = idx % VB;
            sOY[t * VP + y] = t < n ? to_f32(dO[tok_row(a, sl, t0 + t) * V + v0 + y]) : 0.f;
        }
        if (tid < C) sb[tid] = tid < n ? a.beta[tok_row(a, sl, t0 + tid)] : 0.f;
        float *dhS = a.ws.dhS + ci * (K * V);
        for (int idx = tid; idx < K * VB; idx += BW_NTHR) {
            const int x = idx / VB, y = idx % VB;
            dhS[x * V + v0 + y] = sdS[x * VP + y];
        }
        __syncthreads();
        {   // dDelta = Km dS' + P^T dO
            using TL = Tile<C, VB, 4, VB / 16>;
            const TL tl;
            float acc[4][VB / 16] = {};
            mm_acc<C, VB, 4, VB / 16, K, KP, 1, VP, 1>(acc, sKm, sdS, tl.mt, tl.nt);
            mm_acc<C, VB, 4, VB / 16, C, 1, CP, VP, 1>(acc, sP, sOY, tl.mt, tl.nt);
            float *dDl = a.ws.dDl + ci * (C * V);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < VB / 16; ++j) {
                    const int t = tl.row(i), y = tl.col(j);
                    sdD[t * VP + y] = acc[i][j];
                    dDl[t * V + v0 + y] = acc[i][j];
                }
        }
        __syncthreads();
        {   // Y = T^T dDelta, stored as -beta Y under dO
            using TL = Tile<C, VB, 4, VB / 16>;
            const TL tl;
            float acc[4][VB / 16] = {};
            mm_acc<C, VB, 4, VB / 16, C, 1, CP, VP, 1>(acc, sT, sdD, tl.mt, tl.nt);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < VB / 16; ++j) {
                    const int t = tl.row(i), y = tl.col(j);
                    sOY[(C + t) * VP + y] = -sb[t] * acc[i][j];
                }
        }
        __syncthreads();
        {   // dS = Diag(e^{gn}) dS' + [Qp; Kp]^T [dO; -beta Y]
            using TL = Tile<K, VB, K / 16, VB / 16>;
            const TL tl;
            float acc[K / 16][VB / 16] = {};
            mm_acc<K, VB, K / 16, VB / 16, 2 * C, 1, KP, VP, 1>(acc, sQK, sOY, tl.mt, tl.nt);
#pragma unroll
            for (int i = 0; i < K / 16; ++i)
#pragma unroll
                for (int j = 0; j < VB / 16; ++j) {
                    const int x = tl.row(i), y = tl.col(j);
                    sdS[x * VP + y] = sgn[x] * sdS[x * VP + y] + acc[i][j];
                }
        }
    }
    __syncthreads();
    if (a.dS0) {
        for (int idx = tid; idx < K * VB; idx += BW_NTHR) {
            const int x = idx / VB, y = idx % VB;
            a.dS0[((long)sl * K + x) * V + v0 + y] = sdS[x * VP + y];
        }
    }
}

// ---------------------------------------------------------------- 4 vgrad
template <typename DT, int K, int V>
__global__ __launch_bounds__(BW_NTHR) void bwd_vgrad_kernel(BwArgs a)
{
    constexpr int C = BW_C, VB = 16, CP = C + 1, VP = VB + 1;
    extern __shared__ __attribute__((aligned(256))) float sm[];
    float *sS = sm, *sdS = sS + K * VP, *sdO = sdS + K * VP, *sDl = sdO + C * VP;
    float *sdD = sDl + C * VP, *sV = sdD + C * VP, *sT = sV + C * VP, *sb = sT + C * CP;
    const int tid = threadIdx.x;
    const int c = blockIdx.x % a.NC, sl = blockIdx.x / a.NC;
    const int t0 = c * C, n = min(C, a.T - t0);
    const long ci = (long)sl * a.NC + c;
    const DT *v = (const DT *)a.v, *dO = (const DT *)a.d_o;
    DT *dv = (DT *)a.dv;
    const float *hS = a.ws.hS + ci * (K * V), *dhS = a.ws.dhS + ci * (K * V);
    const float *Dl = a.ws.Dl + ci * (C * V), *dDl = a.ws.dDl + ci * (C * V);

    const float *Tm = a.ws.Tm + ci * (C * C);
    for (int idx = tid; idx < C * C; idx += BW_NTHR) sT[(idx / C) * CP + idx % C] = Tm[idx];
    if (tid < C) sb[tid] = tid < n ? a.beta[tok_row(a, sl, t0 + tid)] : 0.f;

    using TCK = Tile<C, K, 4, K / 16>;
    using TCC = Tile<C, C, 4, 4>;
    using TCV = Tile<C, VB, 4, 1>;
    const TCK tk;
    const TCC tc;
    const TCV tv;
    float aQ[4][K / 16] = {}, aKm[4][K / 16] = {}, aWn[4][K / 16] = {};
    float aP[4][4] = {}, aT[4][4] = {};
    float dbv[4] = {0.f, 0.f, 0.f, 0.f};
    float dgn = 0.f;

    for (int v0 = 0; v0 < V; v0 += VB) {
        __syncthreads();
        for (int idx = tid; idx < K * VB; idx += BW_NTHR) {
            const int x = idx / VB, y = idx % VB;
            sS[x * VP + y] = hS[x * V + v0 + y];
            sdS[x * VP + y] = dhS[x * V + v0 + y];
        }
        for (int idx = tid; idx < C * VB; idx += BW_NTHR) {
            const int t = idx / VB, y = idx % VB;
            float o = 0.f, vv = 0.f;
            if (t < n) {
                const long r = tok_row(a, sl, t0 + t);
                o = to_f32(dO[r * V + v0 + y]);
                vv = to_f32(v[r * V + v0 + y]);
            }
            sdO[t * VP + y] = o;
            sV[t * VP + y] = vv;
            sDl[t * VP + y] = Dl[t * V + v0 + y];
            sdD[t * VP + y] = dDl[t * V + v0 + y];
        }
        __syncthreads();
        // dQp += dO S^T, dKm += Delta dS'^T, dWn += dDelta S^T   (C x K, sum over the block)
        mm_acc<C, K, 4, K / 16, VB, VP, 1, 1, VP>(aQ, sdO, sS, tk.mt, tk.nt);
        mm_acc<C, K, 4, K / 16, VB, VP, 1, 1, VP>(aKm, sDl, sdS, tk.mt, tk.nt);
        mm_acc<C, K, 4, K / 16, VB, VP, 1, 1, VP>(aWn, sdD, sS, tk.mt, tk.nt);
        // dP += dO Delta^T, dT += dDelta V^T (beta applied at the end)
        mm_acc<C, C, 4, 4, VB, VP, 1, 1, VP>(aP, sdO, sDl, tc.mt, tc.nt);
        mm_acc<C, C, 4, 4, VB, VP, 1, 1, VP>(aT, sdD, sV, tc.mt, tc.nt);
        {   // Y = T^T dDelta: dv = beta Y, dbeta += rowsum(V * Y)
            float y[4][1] = {};
            mm_acc<C, VB, 4, 1, C, 1, CP, VP, 1>(y, sT, sdD, tv.mt, tv.nt);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = tv.row(i), yy = tv.col(0);
                dbv[i] = fmaf(sV[t * VP + yy], y[i][0], dbv[i]);
                if (t < n) dv[tok_row(a, sl, t0 + t) * V + v0 + yy] = from_f32<DT>(sb[t] * y[i][0]);
            }
        }
        if (tid < K)
            for (int y = 0; y < VB; ++y) dgn = fmaf(sS[tid * VP + y], sdS[tid * VP + y], dgn);
    }

    float *dQp = a.ws.dQp + ci * (C * K), *dKm = a.ws.dKm + ci * (C * K), *dWn = a.ws.dWn + ci * (C * K);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < K / 16; ++j) {
            const int t = tk.row(i), x = tk.col(j);
            dQp[t * K + x] = aQ[i][j];
            dKm[t * K + x] = aKm[i][j];
            dWn[t * K + x] = aWn[i][j];
        }
    float *dP = a.ws.dP + ci * (C * C), *dT = a.ws.dT + ci * (C * C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = tc.row(i), s = tc.col(j);
            dP[t * C + s] = aP[i][j];
            dT[t * C + s] = aT[i][j] * sb[s];
        }
    // rows tv.row(i) are shared by the 16 consecutive lanes with the same tv.mt
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float s = dbv[i];
        s += __shfl_xor(s, 1, 16);
        s += __shfl_xor(s, 2, 16);
        s += __shfl_xor(s, 4, 16);
        s += __shfl_xor(s, 8, 16);
        if (tv.nt == 0) a.ws.dbv[ci * C + tv.row(i)] = s;
    }
    if (tid < K) {
        const float gn = a.ws.gam[ci * (C * K) + (C - 1) * K + tid];
        a.ws.dgn[ci * K + tid] = __expf(gn) * dgn;
    }
}

// ---------------------------------------------------------------- 5 kgrad
template <typename DT, int K, bool CH>
__global__ __launch_bounds__(BW_NTHR) void bwd_kgrad_kernel(BwArgs a)
{
    constexpr int C = BW_C, KP = K + 1, CP = C + 1;
    constexpr int NSPL = BW_NTHR / K;   // threads per key channel in the pair phase
    constexpr int RP = C / NSPL;        // rows per thread there
    extern __shared__ __attribute__((aligned(256))) float sm[];
    // fixed: small arrays, dG (first dT), dP
    float *sb = sm, *sdb = sb + C, *stot = sdb + C, *sdgn = stot + NSPL * K;
    float *sdG = sdgn + NSPL * K, *sdP = sdG + C * CP;
    float *scr = sdP + C * CP;
    // phases 1-2: dWn (then M1), Kp, T;  phase 3: k, gamma, q (unpadded rows)
    float *sWn = scr, *sM = scr, *sKp = scr + C * KP, *sT = sKp + C * KP;
    float *sk = scr, *sg = scr + C * K, *sq = sg + C * K;
    const int tid = threadIdx.x;
    const int c = blockIdx.x % a.NC, sl = blockIdx.x / a.NC;
    const int t0 = c * C, n = min(C, a.T - t0);
    const long ci = (long)sl * a.NC + c;
    const DT *q = (const DT *)a.q, *k = (const DT *)a.k;
    const float *gam = a.ws.gam + ci * (C * K);
    float *Zg = a.ws.dWn + ci * (C * K);   // dWn is replaced by Z once it is in LDS

    for (int idx = tid; idx < C * K; idx += BW_NTHR) {
        const int t = idx / K, x = idx % K;
        const float kv = t < n ? to_f32(k[tok_row(a, sl, t0 + t) * K + x]) : 0.f;
        sKp[t * KP + x] = kv * __expf(gam[idx]);
        sWn[t * KP + x] = Zg[idx];
    }
    {
        const float *Tm = a.ws.Tm + ci * (C * C), *dT = a.ws.dT + ci * (C * C);
        for (int idx = tid; idx < C * C; idx += BW_NTHR) {
            const int t = idx / C, s = idx % C;
            sT[t * CP + s] = Tm[idx];
            sdG[t * CP + s] = dT[idx];
        }
    }
    if (tid < C) {
        sb[tid] = tid < n ? a.beta[tok_row(a, sl, t0 + tid)] : 0.f;
        sdb[tid] = a.ws.dbv[ci * C + tid];
    }
    __syncthreads();
    {   // Z = -T^T dWn (to global, in place of dWn); dbeta += rowsum(Kp * Z)
        using TL = Tile<C, K, 4, K / 16>;
        const TL tl;
        float acc[4][K / 16] = {};
        mm_acc<C, K, 4, K / 16, C, 1, CP, KP, 1>(acc, sT, sWn, tl.mt, tl.nt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tl.row(i);
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < K / 16; ++j) {
                const int x = tl.col(j);
                Zg[t * K + x] = -acc[i][j];
                part = fmaf(sKp[t * KP + x], -acc[i][j], part);
            }
            part += __shfl_xor(part, 1, 16);
            part += __shfl_xor(part, 2, 16);
            part += __shfl_xor(part, 4, 16);
            part += __shfl_xor(part, 8, 16);
            if (tl.nt == 0) sdb[t] += part;
        }
    }
    {   // dT -= dWn (beta Kp)^T
        using TL = Tile<C, C, 4, 4>;
        const TL tl;
        float acc[4][4] = {};
        mm_acc<C, C, 4, 4, K, KP, 1, 1, KP>(acc, sWn, sKp, tl.mt, tl.nt);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = tl.row(i), s = tl.col(j);
                sdG[t * CP + s] -= sb[s] * acc[i][j];
            }
    }
    __syncthreads();
    {   // M1 = T^T dT (over dWn, which is no longer read); dP masked to s <= t
        using TL = Tile<C, C, 4, 4>;
        const TL tl;
        float acc[4][4] = {};
        mm_acc<C, C, 4, 4, C, 1, CP, CP, 1>(acc, sT, sdG, tl.mt, tl.nt);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) sM[tl.row(i) * CP + tl.col(j)] = acc[i][j];
        const float *dP = a.ws.dP + ci * (C * C);
        for (int idx = tid; idx < C * C; idx += BW_NTHR) {
            const int t = idx / C, s = idx % C;
            sdP[t * CP + s] = s <= t ? dP[idx] : 0.f;
        }
    }
    __syncthreads();
    {   // dA = -M1 T^T (strictly lower); dG = diag(beta) dA; dbeta += rowsum(dA * G)
        using TL = Tile<C, C, 4, 4>;
        const TL tl;
        float acc[4][4] = {};
        mm_acc<C, C, 4, 4, C, CP, 1, 1, CP>(acc, sM, sT, tl.mt, tl.nt);
        const float *Gm = a.ws.Gm + ci * (C * C);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tl.row(i);
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = tl.col(j);
                const float da = s < t ? -acc[i][j] : 0.f;
                part = fmaf(da, Gm[t * C + s], part);
                sdG[t * CP + s] = sb[t] * da;
            }
            part += __shfl_xor(part, 1, 16);
            part += __shfl_xor(part, 2, 16);
            part += __shfl_xor(part, 4, 16);
            part += __shfl_xor(part, 8, 16);
            if (tl.nt == 0) sdb[t] += part;
        }
    }
    __syncthreads();
    // phase 3: k, gamma, q by rows, one key channel per thread
    for (int idx = tid; idx < C * K; idx += BW_NTHR) {
        const int t = idx / K;
        float kv = 0.f, qv = 0.f;
        if (t < n) {
            const long r = tok_row(a, sl, t0 + t);
            kv = to_f32(k[r * K + idx % K]);
            qv = to_f32(q[r * K + idx % K]);
        }
        sk[idx] = kv;
        sq[idx] = qv;
        sg[idx] = gam[idx];
    }
    __syncthreads();
    const int x = tid % K, sp = tid / K;
    const int r0 = sp * RP;
    const float gn = sg[(C - 1) * K + x];
    const float *dQp = a.ws.dQp + ci * (C * K), *dKm = a.ws.dKm + ci * (C * K);
    float *dgam = a.ws.dQp + ci * (C * K);   // dQp is replaced by d gamma element by element
    DT *dq = (DT *)a.dq, *dk = (DT *)a.dk;
    float tot = 0.f, dgn_loc = 0.f;
    for (int r = r0; r < r0 + RP; ++r) {
        const float kr = sk[r * K + x], qr = sq[r * K + x], gr = sg[r * K + x];
        float accq = 0.f, acck = 0.f, accs = 0.f;
        for (int s = 0; s <= r; ++s) {          // r as the later token
            const float w = sk[s * K + x] * __expf(gr - sg[s * K + x]);
            accq = fmaf(sdP[r * CP + s], w, accq);
            acck = fmaf(sdG[r * CP + s], w, acck);
        }
        for (int t = r; t < C; ++t) {           // r as the earlier token
            const float e = __expf(sg[t * K + x] - gr);
            accs = fmaf(fmaf(sdG[t * CP + r], sk[t * K + x], sdP[t * CP + r] * sq[t * K + x]), e, accs);
        }
        const float eg = __expf(gr), em = __expf(gn - gr);
        const float dqp = dQp[r * K + x], dkm = dKm[r * K + x], z = Zg[r * K + x] * sb[r];
        const float dqv = fmaf(dqp, eg, accq);
        const float dkv = acck + accs + z * eg + dkm * em;
        const float dgm = qr * accq + kr * (acck - accs) + (dqp * qr + z * kr) * eg - dkm * kr * em;
        dgn_loc = fmaf(dkm * kr, em, dgn_loc);
        if (r < n) {
            const long row = tok_row(a, sl, t0 + r);
            dq[row * K + x] = from_f32<DT>(dqv);
            dk[row * K + x] = from_f32<DT>(dkv);
        }
        dgam[r * K + x] = dgm;
        tot += dgm;
    }
    stot[sp * K + x] = tot;
    sdgn[sp * K + x] = dgn_loc;
    __syncthreads();
    {   // dg = reverse running sum of d gamma, plus the gn terms on the last row
        float run = a.ws.dgn[ci * K + x];
#pragma unroll
        for (int p = 0; p < NSPL; ++p) run += sdgn[p * K + x] + (p > sp ? stot[p * K + x] : 0.f);
        for (int r = r0 + RP - 1; r >= r0; --r) {
            run += dgam[r * K + x];
            if (CH) {
                if (r < n) a.dg[tok_row(a, sl, t0 + r) * K + x] = run;
            } else {
                sk[r * K + x] = run;            // k is no longer read
            }
        }
    }
    if (!CH) {
        __syncthreads();
        if (tid < n) {
            float s = 0.f;
            for (int y = 0; y < K; ++y) s += sk[tid * K + y];
            a.dg[tok_row(a, sl, t0 + tid)] = s;
        }
    }
    if (tid < n) a.dbeta[tok_row(a, sl, t0 + tid)] = sdb[tid];
}

// ---------------------------------------------------------------- host side
template <int K, int V> struct BwLds {
    static constexpr int C = BW_C, KP = K + 1, CP = C + 1, VB = bw_vb(K), VP = VB + 1;
    static constexpr int prep = 4 * (3 * C * KP + 2 * C * CP + C);
    static constexpr int states = 4 * (2 * C * KP + C * CP + K * VP + 2 * C * VP + C + K);
    static constexpr int dstates = 4 * (3 * C * KP + 2 * C * CP + K * VP + 3 * C * VP + C + K);
    static constexpr int vgrad = 4 * (2 * K * 17 + 4 * C * 17 + C * CP + C);
    static constexpr int kscr12 = 2 * C * KP + C * CP, kscr3 = 3 * C * K;
    static constexpr int kgrad = 4 * (2 * C + 2 * (BW_NTHR / K) * K + 2 * C * CP +
                                      (kscr12 > kscr3 ? kscr12 : kscr3));
    static_assert(prep <= 160 * 1024 && states <= 160 * 1024 && dstates <= 160 * 1024 &&
                  vgrad <= 160 * 1024 && kgrad <= 160 * 1024, "LDS budget");
};

template <typename F> static hipError_t set_lds(F *kern, int bytes, bool &done)
{
    if (done) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute((const void *)kern,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done = true;   // benign race: every thread sets the same value
    return e;
}

template <typename DT, int K, int V, bool CH>
static hipError_t launch_bwd(const BwArgs &a, long nslices, hipStream_t st)
{
    using L = BwLds<K, V>;
    static bool s1 = false, s2 = false, s3 = false, s4 = false, s5 = false;
    hipError_t e;
    if ((e = set_lds(bwd_prep_kernel<DT, K, CH>, L::prep, s1)) != hipSuccess) return e;
    if ((e = set_lds(bwd_states_kernel<DT, K, V, CH>, L::states, s2)) != hipSuccess) return e;
    if ((e = set_lds(bwd_dstates_kernel<DT, K, V, CH>, L::dstates, s3)) != hipSuccess) return e;
    if ((e = set_lds(bwd_vgrad_kernel<DT, K, V>, L::vgrad, s4)) != hipSuccess) return e;
    if ((e = set_lds(bwd_kgrad_kernel<DT, K, CH>, L::kgrad, s5)) != hipSuccess) return e;
    const unsigned nch = (unsigned)(nslices * a.NC), nvb = (unsigned)(nslices * (V / L::VB));
    if (nch > 0) {
        hipLaunchKernelGGL((bwd_prep_kernel<DT, K, CH>), dim3(nch), dim3(BW_NTHR), L::prep, st, a);
        hipLaunchKernelGGL((bwd_states_kernel<DT, K, V, CH>), dim3(nvb), dim3(BW_NTHR), L::states, st, a);
    }
    hipLaunchKernelGGL((bwd_dstates_kernel<DT, K, V, CH>), dim3(nvb), dim3(BW_NTHR), L::dstates, st, a);
    if (nch > 0) {
        hipLaunchKernelGGL((bwd_vgrad_kernel<DT, K, V>), dim3(nch), dim3(BW_NTHR), L::vgrad, st, a);
        hipLaunchKernelGGL((bwd_kgrad_kernel<DT, K, CH>), dim3(nch), dim3(BW_NTHR), L::kgrad, st, a);
    }
    return hipGetLastError();
}

template <typename DT, bool CH>
static hipError_t dispatch_bwd(int K, int V, const BwArgs &a, long ns, hipStream_t st)
{
    if (K == 64 && V == 64) return launch_bwd<DT, 64, 64, CH>(a, ns, st);
    if (K == 64 && V == 128) return launch_bwd<DT, 64, 128, CH>(a, ns, st);
    if (K == 128 && V == 64) return launch_bwd<DT, 128, 64, CH>(a, ns, st);
    return launch_bwd<DT, 128, 128, CH>(a, ns, st);
}

// Host entry used by the C ABI after validation (K, V in {64, 128}; B H > 0).
hipError_t chunk_bwd_launch(bool bf16, bool channel, int K, int V, const BwArgs &a, long nslices,
                            hipStream_t st)
{
    if (bf16)
        return channel ? dispatch_bwd<__bf16, true>(K, V, a, nslices, st)
                       : dispatch_bwd<__bf16, false>(K, V, a, nslices, st);
    return channel ? dispatch_bwd<float, true>(K, V, a, nslices, st)
                   : dispatch_bwd<float, false>(K, V, a, nslices, st);
}

} // namespace gdn
