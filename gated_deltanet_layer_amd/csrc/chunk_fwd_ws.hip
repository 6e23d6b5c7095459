// chunk_fwd_ws.hip -- warp-specialised chunkwise forward for bf16 operands and
// the scalar-per-head gate (the prefill hot path of the scalar-gate model).
//
// Same mathematics as chunk_fwd.hip (Atomic-GDN2 model card, section 2.1; the
// chunkwise mode of the MindPattern "Gated DeltaNet" page), with the work of a
// chunk split between two groups of waves that run concurrently:
//
//   chain waves 0-3  own the fp32 state (wave w: value columns 16w..16w+15 of
//                    the workgroup's 64-column block, in MFMA accumulators) and
//                    run chunk c: K+S, Q+S, X = diag(beta)(V - K+S), the block
//                    forward substitution for D, O = Q+S + P D, and
//                    S' = e^{gamma_n} S + K^T (e^{gamma_n - gamma} D).
//   prep waves 4-7   get chunk c+1 ready: stage q, k, k^T, v and the decay
//                    vectors into the other half of a double-buffered LDS set,
//                    then compute the Gram blocks -A (strictly lower), P (lower)
//                    and the 16 x 16 diagonal inverses T_ii, and load chunk c+2
//                    from HBM into registers.
//
// A single workgroup barrier per chunk hands the buffers over.  The prep waves
// also need one barrier among themselves per chunk (staging before Gram); it
// is an LDS arrival counter that only those four waves use, so the chain waves
// never wait for it.  Each SIMD runs one chain wave and one prep wave, so the
// latency-bound prep work (substitution, exponentials, staging) overlaps the
// chain's matrix-core work.
#include "mfma_frag.h"

namespace gdn {

constexpr int WS_T = 64;       // tokens per chunk
constexpr int WS_VB = 64;      // value columns per workgroup
constexpr int WS_NTHR = 512;   // 4 chain waves + 4 prep waves

template <int K> struct WsSmem {
    static constexpr int PAD = 8;                 // bf16 elements = 16 bytes
    static constexpr int LDK = K + PAD;           // [64][K] q and k
    static constexpr int LDC = WS_T + PAD;        // [*][64] v, -A, P
    static constexpr int LDT = WS_T;              // [K][64] k^T (swizzled, unpadded)
    static constexpr int LDD = 16 + PAD;          // [64][16] T_ii
    static constexpr int al(int x) { return (x + 255) & ~255; }
    // one buffer
    static constexpr int oK = 0;
    static constexpr int oQ = oK + WS_T * LDK * 2;
    static constexpr int oKT = oQ + WS_T * LDK * 2;
    static constexpr int oV = oKT + K * LDT * 2;
    static constexpr int oAn = oV + WS_T * LDC * 2;           // rows 16..63 of -A
    static constexpr int oP = oAn + (WS_T - 16) * LDC * 2;
    static constexpr int oTd = oP + WS_T * LDC * 2;
    static constexpr int oBeta = oTd + WS_T * LDD * 2;
    static constexpr int oEg = oBeta + WS_T * 4;               // e^{gamma_t}
    static constexpr int oEgn = oEg + WS_T * 4;                // e^{gamma_n - gamma_t}
    static constexpr int oEgN = oEgn + WS_T * 4;               // e^{gamma_n}
    static constexpr int BUF = al(oEgN + 16);
    static constexpr int kGam = 2 * BUF;                       // prep-private gamma [64]
    static constexpr int kCtr = kGam + WS_T * 4;               // prep arrival counter
    static constexpr int bytes = al(kCtr + 16);
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Barrier among the four prep waves: each wave adds one arrival to an LDS
// counter and waits until the counter reaches `target` (4 per use).  All four
// waves reach every use unconditionally.  The wait is bounded: after ~2^22
// polls it gives up (the results would be wrong, but the kernel still ends).
__device__ __forceinline__ void prep_barrier(unsigned *ctr, unsigned target) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    for (int it = 0; it < (1 << 22); ++it) {
        const unsigned v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((unsigned)__builtin_amdgcn_readfirstlane((int)v) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Gram blocks (i, j), j <= i, per prep wave (same schedule as chunk_fwd.hip):
// one diagonal block each, left-hand fragments reused within a row.
__constant__ const signed char kWsGram[4][3][2] = {
    {{3, 0}, {3, 1}, {0, 0}},
    {{3, 2}, {3, 3}, {-1, -1}},
    {{2, 0}, {2, 1}, {2, 2}},
    {{1, 0}, {1, 1}, {-1, -1}},
};

struct WsArgs {
    const __bf16 *q, *k, *v;
    const float *g, *beta, *S0;
    __bf16 *o;
    float *S_T;
    int T, H, V, nvb;
    int xcd_map;
};

template <int K>
__global__ __launch_bounds__(WS_NTHR, 1) void chunk_fwd_ws_kernel(WsArgs args)
{
    using L = WsSmem<K>;
    constexpr int NT = K / 16;          // 16-row tiles of S
    constexpr int NKB = K / 32;         // 32-wide k blocks over the key dim
    constexpr int EPV = 8;              // bf16 per 16-byte vector
    constexpr int CG = K / EPV;         // vectors per q/k row
    constexpr int RG = 256 / CG;        // row groups over the 256 prep threads
    constexpr int RPT = WS_T / RG;      // rows per prep thread
    constexpr int NVV = WS_T * (WS_VB / EPV) / 256;   // v vectors per prep thread
    using pack_t = typename Pack<__bf16, RPT>::type;
    static_assert(RPT * RG == WS_T, "layout");

    extern __shared__ __attribute__((aligned(256))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int gq = lane >> 4;

    const int T = args.T, H = args.H, V = args.V, nvb = args.nvb;
    int bh, vb;
    {
        const int w = blockIdx.x;
        if (args.xcd_map) {
            const int xcd = w & 7, slot = w >> 3;
            vb = slot % nvb;
            bh = (slot / nvb) * 8 + xcd;
        } else {
            bh = w / nvb;
            vb = w % nvb;
        }
    }
    const int b = bh / args.H, h = bh % args.H;
    const int v0 = vb * WS_VB;
    const long row_base = (long)b * T * H + h;   // row of token 0 in [B*T*H]
    const int nchunks = (T + WS_T - 1) / WS_T;

    auto buf = [&](int c) { return smem + (c & 1) * L::BUF; };
    unsigned *ctr = reinterpret_cast<unsigned *>(smem + L::kCtr);
    if (tid == 0) *ctr = 0u;
    lds_barrier();

    if (wave >= 4) {
        // ============================ prep waves ============================
        const int ptid = tid - 256, pw = wave - 4;
        const int cg = ptid % CG, rg = ptid / CG;
        float *gam = reinterpret_cast<float *>(smem + L::kGam);
        f32x4 pk[RPT], pq[RPT], pv[NVV];
        float pb = 0.f, pg = 0.f;
        auto load = [&](int t0) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int t = t0 + RPT * rg + i;
                f32x4 zk = {0.f, 0.f, 0.f, 0.f}, zq = zk;
                if (t < T) {
                    const long off = (row_base + (long)t * H) * K + cg * EPV;
                    zk = *reinterpret_cast<const f32x4 *>(args.k + off);
                    zq = *reinterpret_cast<const f32x4 *>(args.q + off);
                }
                pk[i] = zk;
                pq[i] = zq;
            }
#pragma unroll
            for (int j = 0; j < NVV; ++j) {
                const int idx = ptid + 256 * j, row = idx / (WS_VB / EPV), cv = idx % (WS_VB / EPV);
                const int t = t0 + row;
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                if (t < T)
                    z = *reinterpret_cast<const f32x4 *>(args.v + (row_base + (long)t * H) * V + v0 + cv * EPV);
                pv[j] = z;
            }
            const bool ok = ptid < WS_T && t0 + ptid < T;
            pg = ok ? args.g[row_base + (long)(t0 + ptid) * H] : 0.f;
            pb = ok ? args.beta[row_base + (long)(t0 + ptid) * H] : 0.f;
        };
        unsigned arrivals = 0;
        // Stage the registers (chunk n) into buffer n&1, load chunk n+1, then
        // compute the Gram blocks and diagonal inverses of chunk n.
        auto prepare = [&](int n) {
            char *B = buf(n);
            __bf16 *sK = reinterpret_cast<__bf16 *>(B + L::oK);
            __bf16 *sQ = reinterpret_cast<__bf16 *>(B + L::oQ);
            __bf16 *sKT = reinterpret_cast<__bf16 *>(B + L::oKT);
            __bf16 *sV = reinterpret_cast<__bf16 *>(B + L::oV);
            __bf16 *sAn = reinterpret_cast<__bf16 *>(B + L::oAn);
            __bf16 *sP = reinterpret_cast<__bf16 *>(B + L::oP);
            __bf16 *sTd = reinterpret_cast<__bf16 *>(B + L::oTd);
            float *sBeta = reinterpret_cast<float *>(B + L::oBeta);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                *reinterpret_cast<f32x4 *>(sK + (RPT * rg + i) * L::LDK + cg * EPV) = pk[i];
                *reinterpret_cast<f32x4 *>(sQ + (RPT * rg + i) * L::LDK + cg * EPV) = pq[i];
            }
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int ch = cg * EPV + e;
                pack_t pt;
#pragma unroll
                for (int i = 0; i < RPT; ++i) pt[i] = reinterpret_cast<const __bf16 *>(&pk[i])[e];
                *reinterpret_cast<pack_t *>(sKT + ch * L::LDT + ((RPT * rg) ^ kmt_swz<EPV>(ch))) = pt;
            }
#pragma unroll
            for (int j = 0; j < NVV; ++j) {
                const int idx = ptid + 256 * j, row = idx / (WS_VB / EPV), cv = idx % (WS_VB / EPV);
                *reinterpret_cast<f32x4 *>(sV + row * L::LDC + cv * EPV) = pv[j];
            }
            if (pw == 0) {
                // running sum of g over the chunk (lane = token) and its decays
                const float x = wave_inclusive_sum(pg);
                const float gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
                gam[lane] = x;
                reinterpret_cast<float *>(B + L::oEg)[lane] = __expf(x);
                reinterpret_cast<float *>(B + L::oEgn)[lane] = __expf(gn - x);
                if (lane == 0) reinterpret_cast<float *>(B + L::oEgN)[0] = __expf(gn);
                sBeta[lane] = pb;
            }
            if (n + 1 < nchunks) load((n + 1) * WS_T);
            arrivals += 4;
            prep_barrier(ctr, arrivals);

            // Gram blocks on the static schedule
            Frag<__bf16> aK[NKB], aQ[NKB];
            int cur_i = -1;
#pragma unroll
            for (int pp = 0; pp < 3; ++pp) {
                const int i = kWsGram[pw][pp][0], j = kWsGram[pw][pp][1];
                if (i < 0) break;
                if (i != cur_i) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        aK[kb] = lds_frag(sK, L::LDK, 16 * i, 32 * kb);
                        aQ[kb] = lds_frag(sQ, L::LDK, 16 * i, 32 * kb);
                    }
                    cur_i = i;
                }
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = accA;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const Frag<__bf16> fr = lds_frag(sK, L::LDK, 16 * j, 32 * kb);
                    accA = mma(accA, aK[kb], fr);
                    accP = mma(accP, aQ[kb], fr);
                }
                // rows t = 16i + 4gq + e, column s = 16j + r16
                const int s = 16 * j + r16;
                const f32x4 bt = *reinterpret_cast<const f32x4 *>(sBeta + 16 * i + 4 * gq);
                const f32x4 gt = *reinterpret_cast<const f32x4 *>(gam + 16 * i + 4 * gq);
                const float gs = gam[s];
                f32x4 a, p;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * i + 4 * gq + e;
                    const float dec = (s <= t) ? __expf(gt[e] - gs) : 0.f;
                    a[e] = (s < t) ? bt[e] * accA[e] * dec : 0.f;
                    p[e] = accP[e] * dec;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * i + 4 * gq + e;
                    sP[t * L::LDC + s] = (__bf16)p[e];
                    if (j < i) sAn[(t - 16) * L::LDC + s] = (__bf16)(-a[e]);
                }
                if (j == i) {
                    // column r16 of T_ii = (I + A_ii)^{-1} by forward substitution;
                    // A[r'][r] is in lane 16*(r'/4) + r, element r'%4 (readlane)
                    float x[16];
#pragma unroll
                    for (int rr = 0; rr < 16; ++rr) x[rr] = (rr == r16) ? 1.f : 0.f;
#pragma unroll
                    for (int r = 0; r < 15; ++r)
#pragma unroll
                        for (int r2 = r + 1; r2 < 16; ++r2)
                            x[r2] -= __int_as_float(__builtin_amdgcn_readlane(
                                         __float_as_int(a[r2 & 3]), 16 * (r2 >> 2) + r)) * x[r];
                    if (gq == 0) {
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr)
                            sTd[(16 * i + rr) * L::LDD + r16] = (__bf16)x[rr];
                    }
                }
            }
        };

        if (nchunks > 0) {
            load(0);
            prepare(0);
            lds_barrier();
        }
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) prepare(c + 1);
            lds_barrier();
        }
        return;
    }

    // ============================= chain waves =============================
    const int vcol = 16 * wave + r16;   // this lane's column inside the block
    f32x4 S_acc[NT];
    {
        const float *S0 = args.S0 ? args.S0 + (long)bh * K * V : nullptr;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S_acc[ct][e] = S0 ? S0[(16 * ct + 4 * gq + e) * V + v0 + vcol] : 0.f;
    }
    if (nchunks > 0) lds_barrier();     // chunk 0 is ready

    for (int c = 0; c < nchunks; ++c) {
        char *B = buf(c);
        const __bf16 *sK = reinterpret_cast<const __bf16 *>(B + L::oK);
        const __bf16 *sQ = reinterpret_cast<const __bf16 *>(B + L::oQ);
        const __bf16 *sKT = reinterpret_cast<const __bf16 *>(B + L::oKT);
        __bf16 *sV = reinterpret_cast<__bf16 *>(B + L::oV);
        const __bf16 *sAn = reinterpret_cast<const __bf16 *>(B + L::oAn);
        const __bf16 *sP = reinterpret_cast<const __bf16 *>(B + L::oP);
        const __bf16 *sTd = reinterpret_cast<const __bf16 *>(B + L::oTd);
        const float *sBeta = reinterpret_cast<const float *>(B + L::oBeta);
        const float *sEg = reinterpret_cast<const float *>(B + L::oEg);
        const float *sEgn = reinterpret_cast<const float *>(B + L::oEgn);
        const float egN = reinterpret_cast<const float *>(B + L::oEgN)[0];

        // K+ S and Q+ S
        f32x4 KS[4], QS[4];
        {
            Frag<__bf16> Sb[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) Sb[kb] = reg_frag<__bf16>(S_acc[2 * kb], S_acc[2 * kb + 1]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = ak;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    ak = mma(ak, lds_frag(sK, L::LDK, 16 * rt, 32 * kb), Sb[kb]);
                    aq = mma(aq, lds_frag(sQ, L::LDK, 16 * rt, 32 * kb), Sb[kb]);
                }
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(sEg + 16 * rt + 4 * gq);
                KS[rt] = ak * eg;
                QS[rt] = aq * eg;
            }
        }
        // X = diag(beta) (V - K+ S)
        f32x4 X[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 bt = *reinterpret_cast<const f32x4 *>(sBeta + 16 * rt + 4 * gq);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                X[rt][e] = bt[e] * ((float)sV[(16 * rt + 4 * gq + e) * L::LDC + vcol] - KS[rt][e]);
        }
        // (I + A) D = X by block forward substitution (sAn holds -A, rows from 16)
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 D[4];
        D[0] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 0, 0), reg_frag<__bf16>(X[0], z));
        f32x4 Y = mma_lo(X[1], lds_frag_lo(sAn, L::LDC, 0, 0), reg_frag<__bf16>(D[0], z));
        D[1] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 16, 0), reg_frag<__bf16>(Y, z));
        const Frag<__bf16> Df0 = reg_frag<__bf16>(D[0], D[1]);
        Y = mma(X[2], lds_frag(sAn, L::LDC, 16, 0), Df0);
        f32x4 Y3 = mma(X[3], lds_frag(sAn, L::LDC, 32, 0), Df0);
        D[2] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 32, 0), reg_frag<__bf16>(Y, z));
        Y3 = mma_lo(Y3, lds_frag_lo(sAn, L::LDC, 32, 32), reg_frag<__bf16>(D[2], z));
        D[3] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 48, 0), reg_frag<__bf16>(Y3, z));
        const Frag<__bf16> Df1 = reg_frag<__bf16>(D[2], D[3]);

        // O = Q+ S + P D
        f32x4 O[4];
        O[0] = mma_lo(QS[0], lds_frag_lo(sP, L::LDC, 0, 0), Df0);
        O[1] = mma(QS[1], lds_frag(sP, L::LDC, 16, 0), Df0);
        O[2] = mma(QS[2], lds_frag(sP, L::LDC, 32, 0), Df0);
        O[2] = mma_lo(O[2], lds_frag_lo(sP, L::LDC, 32, 32), Df1);
        O[3] = mma(QS[3], lds_frag(sP, L::LDC, 48, 0), Df0);
        O[3] = mma(O[3], lds_frag(sP, L::LDC, 48, 32), Df1);
        if (args.o) {
            // through this wave's own v columns (already consumed) for row stores
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sV[(16 * rt + 4 * gq + e) * L::LDC + vcol] = (__bf16)O[rt][e];
            asm volatile("" ::: "memory");
            const int t = c * WS_T + lane;
            if (t < T) {
                const f32x4 *src = reinterpret_cast<const f32x4 *>(sV + lane * L::LDC + 16 * wave);
                f32x4 *dst = reinterpret_cast<f32x4 *>(args.o + (row_base + (long)t * H) * V + v0 + 16 * wave);
                dst[0] = src[0];
                dst[1] = src[1];
            }
        }

        // S' = e^{gamma_n} S + K^T (e^{gamma_n - gamma} D)
        f32x4 Dt[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            Dt[rt] = D[rt] * *reinterpret_cast<const f32x4 *>(sEgn + 16 * rt + 4 * gq);
        const Frag<__bf16> Ef0 = reg_frag<__bf16>(Dt[0], Dt[1]), Ef1 = reg_frag<__bf16>(Dt[2], Dt[3]);
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            S_acc[ct] *= egN;
            S_acc[ct] = mma(S_acc[ct], lds_frag_kmt<EPV>(sKT, L::LDT, 16 * ct, 0), Ef0);
            S_acc[ct] = mma(S_acc[ct], lds_frag_kmt<EPV>(sKT, L::LDT, 16 * ct, 32), Ef1);
        }
        lds_barrier();
    }

    if (args.S_T) {
        float *ST = args.S_T + (long)bh * K * V;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) ST[(16 * ct + 4 * gq + e) * V + v0 + vcol] = S_acc[ct][e];
    }
}

template <int K>
static hipError_t launch_ws(const WsArgs &a, long nwg, hipStream_t stream)
{
    using L = WsSmem<K>;
    static bool attr_set = false;  // benign race: every thread sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_fwd_ws_kernel<K>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(chunk_fwd_ws_kernel<K>, dim3((unsigned)nwg), dim3(WS_NTHR), L::bytes, stream, a);
    return hipGetLastError();
}

// Host entry for bf16 operands with the scalar gate (K = 64 or 128).
hipError_t chunk_fwd_ws_launch(int K, const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *S0, void *o, float *S_T, int B,
                               int T, int H, int V, hipStream_t st)
{
    WsArgs a;
    a.q = (const __bf16 *)q; a.k = (const __bf16 *)k; a.v = (const __bf16 *)v;
    a.g = g; a.beta = beta; a.S0 = S0; a.o = (__bf16 *)o; a.S_T = S_T;
    a.T = T; a.H = H; a.V = V;
    a.nvb = V / WS_VB;
    const long bhn = (long)B * H;
    a.xcd_map = (a.nvb > 1 && bhn % 8 == 0) ? 1 : 0;
    const long nwg = bhn * a.nvb;
    return K == 64 ? launch_ws<64>(a, nwg, st) : launch_ws<128>(a, nwg, st);
}

} // namespace gdn
