// chunk_fwd.hip -- chunkwise forward of the gated delta rule on gfx950.
//
// Recurrence (Atomic-GDN2 model card, section 2.1), per (batch, head):
//   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
//   o_t = S_t^T q_t,   alpha_t = exp(g_t).
// The chunkwise mode computes the same mathematics as the token recurrence
// (MindPattern "Gated DeltaNet" page, finding of 2026-07-29).  For a chunk of n
// tokens entering with state S (K x V), with gamma_t the running sum of g inside
// the chunk (per key channel; a scalar gate is broadcast):
//   A_ts = beta_t sum_c k_tc k_sc e^{gamma_tc - gamma_sc}   (s < t, else 0)
//   P_ts =        sum_c q_tc k_sc e^{gamma_tc - gamma_sc}   (s <= t, else 0)
//   (I + A) D = diag(beta) (V - K+ S),  K+_t = e^{gamma_t} k_t
//   O  = Q+ S + P D,                    Q+_t = e^{gamma_t} q_t
//   S' = Diag(e^{gamma_n}) S + K-^T D,  K-_t = e^{gamma_n - gamma_t} k_t
// I + A is unit lower triangular.  D is found by block forward substitution
// over 16-token blocks: D_i = T_ii (X_i - sum_{j<i} A_ij D_j), with T_ii the
// inverse of the 16 x 16 diagonal block of I + A.
//
// Work split.  One workgroup of 4 waves owns one (b, h, 64-column block of V)
// and walks the chunks of that sequence in order; every column of S evolves on
// its own, so column blocks need no communication.  Wave w owns value columns
// 16w..16w+15 of the block and keeps that K x 16 slice of S in registers, in
// the MFMA accumulator layout, for the whole sequence; the state products
// chain through registers (operand layout: gdn_common.h).  The K-only work of a
// chunk (Gram blocks, diagonal inverses) is split over the 4 waves on a static
// schedule; each wave inverts the diagonal block it computed, so no barrier
// separates the two.  The next chunk's q/k/v/g/beta are loaded into registers
// while the current chunk computes.  Three workgroup barriers per chunk
// (five with the per-channel gate).
//
// Per-key-channel gate: the decay sits inside the contractions of A and P.  It
// is split at 16-token block boundaries: with lambda the running sum of g from
// the start of the token's 16-token block and R_b the running sum up to the
// start of block b,
//   e^{gamma_t - gamma_s} = e^{lambda_t} * e^{R_i - R_j} * e^{-lambda_s}
// for t in block i and s in block j <= i.  With g in [-5, 0], |lambda| <= 80,
// so e^{-lambda} stays below 5.6e34, inside the fp32/bf16 range; the middle
// factor is <= 1.  This is why the gate domain is bounded (the card's
// section 2.1 says the bound comes from the kernel, not from the model).
#include "mfma_frag.h"
#include "prologue_ops.h"
#include "prologue.h"

namespace gdn {

constexpr int CH_T = 64;   // tokens per chunk
constexpr int VBLK = 64;   // value columns per workgroup
constexpr int NTHR = 256;

// ---------------------------------------------------------------------------
// LDS layout (bytes).  Operand arrays carry a 16-byte row pad.
template <typename OT, int K, bool CH, bool PRO = false> struct Smem {
    static constexpr int PAD = 16 / (int)sizeof(OT);
    static constexpr int LDK = K + PAD;          // [64][K] operand arrays
    static constexpr int LDC = CH_T + PAD;       // [*][64] operand arrays
    static constexpr int LDD = 16 + PAD;         // [64][16] diagonal inverses
    static constexpr int LDA = 20;               // [16][16] fp32 scratch (+4 pad)
    static constexpr int E = (int)sizeof(OT);
    static constexpr int align(int x) { return (x + 255) & ~255; }
    static constexpr int kK = 0;
    static constexpr int kQ = align(kK + CH_T * LDK * E);
    static constexpr int kKI = align(kQ + CH_T * LDK * E);
    static constexpr int kKmT = align(kKI + (CH ? CH_T * LDK * E : 0));
    static constexpr int kV = align(kKmT + K * LDC * E);
    static constexpr int kO = align(kV + CH_T * LDC * E);
    static constexpr int kAn = align(kO + CH_T * LDC * E);
    static constexpr int kP = align(kAn + CH_T * LDC * E);
    static constexpr int kTd = align(kP + CH_T * LDC * E);
    static constexpr int kAd = align(kTd + CH_T * LDD * E);      // [4 waves][16][LDA] fp32
    static constexpr int kBeta = align(kAd + 4 * 16 * LDA * 4);
    static constexpr int kG = kBeta + CH_T * 4;                   // scalar g [64]
    static constexpr int kWg = kG + CH_T * 4;                     // write gate [64]
    static constexpr int kW = kWg + CH_T * 4;                     // [4 waves][3][64]
    static constexpr int kLam = align(kW + 4 * 3 * CH_T * 4);     // channel: [4][K]
    static constexpr int kER = kLam + (CH ? 4 * K * 4 : 0);       // [5][K] e^{R_b}
    static constexpr int kFP = kER + (CH ? 5 * K * 4 : 0);        // [6][K] e^{R_i - R_j}
    // fused prologue: convolution taps of this head's q and k channels and of
    // the workgroup's value columns, [K][4], [K][4], [VBLK][4] floats
    static constexpr int kTap = align(kFP + (CH ? 6 * K * 4 : 0));
    static constexpr int bytes = align(kTap + (PRO ? (2 * K + VBLK) * 16 : 0));
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Off-diagonal 16-token block pair (i, j), j < i -> index of its factor row.
__device__ __forceinline__ int pair_idx(int i, int j) { return i * (i - 1) / 2 + j; }

struct ChunkArgs {
    const void *q, *k, *v;
    const float *g, *beta, *S0;
    const float *wgate;   // decoupled write gate, or nullptr (beta writes too)
    void *o;
    float *S_T;
    int B, T, H, V, nvb;
    int xcd_map;  // 1: place the column blocks of one head on one XCD
    // Fused prologue: q, k, v, g and beta above are then the raw projections
    // (q_raw, k_raw, v_raw, g_raw, b_raw); taps [H*K,4], [H*K,4], [H*V,4]; carried
    // convolution states [B,3,H*K] / [B,3,H*V] in the storage type (null: zeros
    // in, not written out; an output never overlaps an input).
    const float *w_q, *w_k, *w_v;
    const void *cs_q, *cs_k, *cs_v;
    void *cs_q_out, *cs_k_out, *cs_v_out;
    float cap;
    int silu;
};

// PRO: the prologue (kernel-4 causal convolution, optional SiLU, q/k L2 norm,
// g = -min(softplus(g_raw), cap), beta = sigmoid(b_raw)) runs in the load stage:
// each thread also loads the three raw rows before its first row (from the
// carried state before the sequence), and transforms its registers in fp32
// before they are staged, so the transformed q, k, v, g and beta never leave
// the chip.  The arithmetic is that of the standalone prologue kernel, token by
// token and in the same order.
template <typename DT, int K, bool CH, bool PRO = false>
__global__ __launch_bounds__(NTHR, 1) void chunk_fwd_kernel(ChunkArgs args)
{
    using OT = DT;                         // MFMA operand type
    using L = Smem<OT, K, CH, PRO>;
    constexpr int NT = K / 16;             // 16-row tiles of S
    constexpr int NKB = K / 32;            // 32-wide k blocks over the key dim
    constexpr int EPV = 16 / (int)sizeof(DT);            // elements per 16-B vector
    constexpr int CG = K / EPV;                          // vectors per q/k row
    constexpr int RG = NTHR / CG;                        // row groups
    constexpr int RPT = CH_T / RG;                       // rows per thread (q/k)
    constexpr int VPRV = VBLK / EPV;                     // vectors per v/o row
    constexpr int NVV = CH_T * VPRV / NTHR;              // v/o vectors per thread
    constexpr int CPT = K / 64;                          // channel-gate prep: channels per thread
    using vec_t = f32x4;                                 // 16-byte transport type
    using pack_t = typename Pack<DT, RPT>::type;
    static_assert(RPT * RG == CH_T && NVV >= 1, "layout");

    extern __shared__ __attribute__((aligned(256))) char smem[];
    OT *sK = reinterpret_cast<OT *>(smem + L::kK);
    OT *sQ = reinterpret_cast<OT *>(smem + L::kQ);
    OT *sKI = reinterpret_cast<OT *>(smem + L::kKI);
    OT *sKmT = reinterpret_cast<OT *>(smem + L::kKmT);
    OT *sV = reinterpret_cast<OT *>(smem + L::kV);
    DT *sO = reinterpret_cast<DT *>(smem + L::kO);
    OT *sAn = reinterpret_cast<OT *>(smem + L::kAn);
    OT *sP = reinterpret_cast<OT *>(smem + L::kP);
    OT *sTd = reinterpret_cast<OT *>(smem + L::kTd);
    float *sBeta = reinterpret_cast<float *>(smem + L::kBeta);
    float *sG = reinterpret_cast<float *>(smem + L::kG);
    float *sWg = reinterpret_cast<float *>(smem + L::kWg);
    float *sLam = reinterpret_cast<float *>(smem + L::kLam);
    float *sER = reinterpret_cast<float *>(smem + L::kER);
    float *sFP = reinterpret_cast<float *>(smem + L::kFP);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform copy
    const int r16 = lane & 15;
    const int gq = lane >> 4;
    float *sW = reinterpret_cast<float *>(smem + L::kW) + wave * 3 * CH_T;       // wave-private
    float *wGam = sW, *wEg = sW + CH_T, *wEgn = sW + 2 * CH_T;

    // workgroup -> (b*H + h, column block)
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
    const int b = bh / H, h = bh % H;
    const int v0 = vb * VBLK;
    const int vcol = 16 * wave + r16;      // this lane's column inside the block

    const DT *qg = static_cast<const DT *>(args.q);
    const DT *kg = static_cast<const DT *>(args.k);
    const DT *vg = static_cast<const DT *>(args.v);
    DT *og = static_cast<DT *>(args.o);
    const long row_base = (long)b * T * H + h;   // row of token 0 in [B*T*H]

    // State slice in accumulator layout: S_acc[ct][e] = S[16ct + 4gq + e][v0 + vcol].
    f32x4 S_acc[NT];
    {
        const float *S0 = args.S0 ? args.S0 + (long)bh * K * V : nullptr;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S_acc[ct][e] = S0 ? S0[(16 * ct + 4 * gq + e) * V + v0 + vcol] : 0.f;
    }

    // ---- prefetch registers for one chunk ----
    // q/k: thread (cg = tid % CG, rg = tid / CG) loads rows RPT*rg .. +RPT-1,
    // 16 bytes at column cg*EPV; v: NVV 16-byte vectors; channel g: thread
    // (blk = tid / 64, cp = tid % 64) loads CPT channels of its 16 tokens.
    const int cg = tid % CG, rg = tid / CG;
    // PRO: raw rows with the three before them (index 0..2), else the rows only
    constexpr int HQ = PRO ? 3 : 0;
    vec_t pk[RPT + HQ], pq[RPT + HQ], pv[NVV][1 + HQ];
    float pgc[CH ? 16 : 1][CH ? CPT : 1];
    float pb = 0.f, pgs = 0.f, pw = 0.f;
    const float *wsrc = args.wgate ? args.wgate : args.beta;
    // carried-state rows (token t < 0 of the sequence): row 3 + t of [B,3,H*D]
    const DT *csq = static_cast<const DT *>(args.cs_q), *csk = static_cast<const DT *>(args.cs_k);
    const DT *csv = static_cast<const DT *>(args.cs_v);
    auto load_chunk = [&](int t0) {
#pragma unroll
        for (int i = 0; i < RPT + HQ; ++i) {
            const int t = t0 + RPT * rg + i - HQ;
            vec_t zk = {0.f, 0.f, 0.f, 0.f}, zq = zk;
            if (t >= 0 && t < T) {
                const long off = (row_base + (long)t * H) * K + cg * EPV;
                zk = *reinterpret_cast<const vec_t *>(kg + off);
                zq = *reinterpret_cast<const vec_t *>(qg + off);
            } else if (PRO && t < 0) {
                const long off = ((long)b * 3 + 3 + t) * H * K + h * K + cg * EPV;
                if (csk) zk = *reinterpret_cast<const vec_t *>(csk + off);
                if (csq) zq = *reinterpret_cast<const vec_t *>(csq + off);
            }
            pk[i] = zk;
            pq[i] = zq;
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int idx = tid + NTHR * j, row = idx / VPRV, cv = idx % VPRV;
#pragma unroll
            for (int i = 0; i <= HQ; ++i) {
                const int t = t0 + row + i - HQ;
                vec_t z = {0.f, 0.f, 0.f, 0.f};
                if (t >= 0 && t < T)
                    z = *reinterpret_cast<const vec_t *>(vg + (row_base + (long)t * H) * V + v0 + cv * EPV);
                else if (PRO && t < 0 && csv)
                    z = *reinterpret_cast<const vec_t *>(csv + ((long)b * 3 + 3 + t) * H * V + h * V + v0 + cv * EPV);
                pv[j][i] = z;
            }
        }
        if constexpr (!CH)
            pgs = (tid < CH_T && t0 + tid < T) ? args.g[row_base + (long)(t0 + tid) * H] : 0.f;
        pb = (tid < CH_T && t0 + tid < T) ? args.beta[row_base + (long)(t0 + tid) * H] : 0.f;
        pw = (tid < CH_T && t0 + tid < T) ? wsrc[row_base + (long)(t0 + tid) * H] : 0.f;
    };
    auto load_gate = [&](int t0) {  // per-channel gate, in the prep mapping
        if constexpr (CH) {
            const int blk = tid >> 6, cp = tid & 63;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                const int t = t0 + 16 * blk + tt;
#pragma unroll
                for (int ci = 0; ci < CPT; ++ci)
                    pgc[tt][ci] = (t < T) ? args.g[(row_base + (long)t * H) * K + cp * CPT + ci] : 0.f;
            }
        }
    };

    const int nchunks = (T + CH_T - 1) / CH_T;
    if (nchunks > 0) {
        load_chunk(0);
        load_gate(0);
    }

    // PRO: the taps in LDS; the staged values of a chunk are the prologue's
    // outputs, computed from the raw registers in fp32.
    float *sTap = reinterpret_cast<float *>(smem + L::kTap);
    if constexpr (PRO) {
        for (int i = tid; i < 2 * K + VBLK; i += NTHR) {
            const float *src = i < K ? args.w_q + ((long)h * K + i) * 4
                             : i < 2 * K ? args.w_k + ((long)h * K + i - K) * 4
                                         : args.w_v + ((long)h * V + v0 + i - 2 * K) * 4;
            *reinterpret_cast<f32x4 *>(sTap + 4 * i) = *reinterpret_cast<const f32x4 *>(src);
        }
        lds_barrier();
    }
    const bool silu = args.silu != 0;
    // q or k rows of this thread: convolution, activation, L2 norm over the
    // head's K channels (the CG lanes of a row reduce with shuffles), rows past
    // the sequence zeroed
    auto qk_prologue = [&](const vec_t (&raw)[RPT + HQ], const float *taps, vec_t (&out)[RPT],
                           int t0) {
        float y[RPT][EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
            const f32x4 w = *reinterpret_cast<const f32x4 *>(taps + (cg * EPV + e) * 4);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float v = pr_conv4(w, to_f32(reinterpret_cast<const DT *>(&raw[i])[e]),
                                         to_f32(reinterpret_cast<const DT *>(&raw[i + 1])[e]),
                                         to_f32(reinterpret_cast<const DT *>(&raw[i + 2])[e]),
                                         to_f32(reinterpret_cast<const DT *>(&raw[i + 3])[e]));
                y[i][e] = silu ? pr_silu(v) : v;
            }
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < EPV; ++e) ss = fmaf(y[i][e], y[i][e], ss);
#pragma unroll
            for (int off = 1; off < CG; off <<= 1) ss += __shfl_xor(ss, off, CG);
            const float rn = (t0 + RPT * rg + i < T) ? pr_rnorm(ss) : 0.f;
            DT *o = reinterpret_cast<DT *>(&out[i]);
#pragma unroll
            for (int e = 0; e < EPV; ++e) o[e] = from_f32<DT>(y[i][e] * rn);
        }
    };
    vec_t xk[RPT], xq[RPT], xv[NVV];   // the values staged for the chunk
    auto stage_values = [&](int t0) {
        if constexpr (!PRO) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                xk[i] = pk[i];
                xq[i] = pq[i];
            }
#pragma unroll
            for (int j = 0; j < NVV; ++j) xv[j] = pv[j][0];
        } else {
            qk_prologue(pq, sTap, xq, t0);
            qk_prologue(pk, sTap + 4 * K, xk, t0);
#pragma unroll
            for (int j = 0; j < NVV; ++j) {
                const int idx = tid + NTHR * j, row = idx / VPRV, cv = idx % VPRV;
                const bool live = t0 + row < T;
                DT *o = reinterpret_cast<DT *>(&xv[j]);
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const f32x4 w = *reinterpret_cast<const f32x4 *>(sTap + (2 * K + cv * EPV + e) * 4);
                    const float v = pr_conv4(w, to_f32(reinterpret_cast<const DT *>(&pv[j][0])[e]),
                                             to_f32(reinterpret_cast<const DT *>(&pv[j][1])[e]),
                                             to_f32(reinterpret_cast<const DT *>(&pv[j][2])[e]),
                                             to_f32(reinterpret_cast<const DT *>(&pv[j][3])[e]));
                    o[e] = from_f32<DT>(live ? (silu ? pr_silu(v) : v) : 0.f);
                }
            }
        }
    };

    // Write the staged outputs of the chunk at t0 (rows < nvalid) from sO to o.
    auto flush_o = [&](int t0, int nvalid) {
        if (!og) return;
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int idx = tid + NTHR * j, row = idx / VPRV, cv = idx % VPRV;
            if (row < nvalid)
                *reinterpret_cast<vec_t *>(og + (row_base + (long)(t0 + row) * H) * V + v0 + cv * EPV) =
                    *reinterpret_cast<const vec_t *>(sO + row * L::LDC + cv * EPV);
        }
    };

    for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * CH_T;

        // ---- stage the prefetched chunk into LDS (and flush the last outputs) ----
        if (c > 0) flush_o(t0 - CH_T, CH_T);
        stage_values(t0);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            *reinterpret_cast<vec_t *>(sK + (RPT * rg + i) * L::LDK + cg * EPV) = xk[i];
            *reinterpret_cast<vec_t *>(sQ + (RPT * rg + i) * L::LDK + cg * EPV) = xq[i];
        }
        if constexpr (!CH) {
            // K^T (the scalar decay is applied to D instead): for each channel of
            // this thread's vector, RPT consecutive tokens in one packed write.
#pragma unroll
            for (int e = 0; e < EPV; ++e) {
                const int ch = cg * EPV + e;
                pack_t pk_t;
#pragma unroll
                for (int i = 0; i < RPT; ++i) pk_t[i] = reinterpret_cast<const DT *>(&xk[i])[e];
                *reinterpret_cast<pack_t *>(sKmT + ch * L::LDC + ((RPT * rg) ^ kmt_swz<EPV>(ch))) = pk_t;
            }
        }
#pragma unroll
        for (int j = 0; j < NVV; ++j) {
            const int idx = tid + NTHR * j, row = idx / VPRV, cv = idx % VPRV;
            *reinterpret_cast<vec_t *>(sV + row * L::LDC + cv * EPV) = xv[j];
        }
        if (tid < CH_T) {
            const bool live = t0 + tid < T;
            const float bv = PRO ? (live ? pr_sigmoid(pb) : 0.f) : pb;
            sBeta[tid] = bv;
            sWg[tid] = PRO ? bv : pw;
            if (!CH) sG[tid] = PRO ? (live ? pr_gate(pgs, args.cap) : 0.f) : pgs;
        }
        lds_barrier();

        // ---- gate preparation ----
        float egN = 1.f;       // scalar gate: e^{gamma_n}
        if constexpr (!CH) {
            if (c + 1 < nchunks) load_chunk(t0 + CH_T);
            // every wave scans g itself (lane = token) into its private vectors
            const float x = wave_inclusive_sum(sG[lane]);
            const float gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
            wGam[lane] = x;
            wEg[lane] = __expf(x);
            wEgn[lane] = __expf(gn - x);
            egN = __expf(gn);
        } else {
            // thread -> 16-token block blk, channels cp*CPT .. +CPT-1
            const int blk = tid >> 6, cp = tid & 63;
            float kraw[16][CPT], lamv[16][CPT];
#pragma unroll
            for (int ci = 0; ci < CPT; ++ci) {
                const int ch = cp * CPT + ci;
                float lam = 0.f;
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) {
                    const int t = 16 * blk + tt;
                    lam += PRO ? (t0 + t < T ? pr_gate(pgc[tt][ci], args.cap) : 0.f) : pgc[tt][ci];
                    const float el = __expf(lam);
                    const float eil = __expf(-lam);
                    const float kv = to_f32(sK[t * L::LDK + ch]);
                    const float qv = to_f32(sQ[t * L::LDK + ch]);
                    sK[t * L::LDK + ch] = from_f32<OT>(kv * el);
                    sQ[t * L::LDK + ch] = from_f32<OT>(qv * el);
                    sKI[t * L::LDK + ch] = from_f32<OT>(kv * eil);
                    kraw[tt][ci] = kv;
                    lamv[tt][ci] = lam;
                }
                sLam[blk * K + ch] = lam;
            }
            if (c + 1 < nchunks) {
                load_chunk(t0 + CH_T);
                load_gate(t0 + CH_T);
            }
            lds_barrier();
#pragma unroll
            for (int ci = 0; ci < CPT; ++ci) {
                const int ch = cp * CPT + ci;
                float Rb[5];
                Rb[0] = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) Rb[i + 1] = Rb[i] + sLam[i * K + ch];
                const float base = Rb[4] - Rb[blk];
                const int swz = kmt_swz<EPV>(ch);
#pragma unroll
                for (int tt = 0; tt < 16; ++tt)
                    sKmT[ch * L::LDC + ((16 * blk + tt) ^ swz)] =
                        from_f32<OT>(kraw[tt][ci] * __expf(base - lamv[tt][ci]));
                if (blk == 0) {
#pragma unroll
                    for (int i = 0; i < 5; ++i) sER[i * K + ch] = __expf(Rb[i]);
#pragma unroll
                    for (int i = 1; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < i; ++j)
                            sFP[pair_idx(i, j) * K + ch] = __expf(Rb[i] - Rb[j]);
                }
            }
            lds_barrier();
        }

        // ---- Gram blocks and diagonal inverses (static per-wave schedule) ----
        {
            const OT *rhs = CH ? sKI : sK;
            Frag<OT> aK[NKB], aQ[NKB];
            int cur_i = -1;
#pragma unroll
            for (int pp = 0; pp < 3; ++pp) {
                int i, j;
                gram_block(wave_u, pp, i, j);
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
                    Frag<OT> fr = lds_frag(rhs, L::LDK, 16 * j, 32 * kb);
                    if (CH && j < i) fr = scale_frag(fr, sFP + pair_idx(i, j) * K, 32 * kb);
                    accA = mma(accA, aK[kb], fr);
                    accP = mma(accP, aQ[kb], fr);
                }
                // rows t = 16i + 4gq + e, column s = 16j + r16
                const int s = 16 * j + r16;
                const f32x4 bt = *reinterpret_cast<const f32x4 *>(sBeta + 16 * i + 4 * gq);
                f32x4 a, p;
                f32x4 gt = {0.f, 0.f, 0.f, 0.f};
                float gs = 0.f;
                if constexpr (!CH) {
                    gt = *reinterpret_cast<const f32x4 *>(wGam + 16 * i + 4 * gq);
                    gs = wGam[s];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * i + 4 * gq + e;
                    const float dec = CH ? 1.f : ((s <= t) ? __expf(gt[e] - gs) : 0.f);
                    a[e] = (s < t) ? bt[e] * accA[e] * dec : 0.f;
                    p[e] = (s <= t) ? accP[e] * dec : 0.f;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * i + 4 * gq + e;
                    sP[t * L::LDC + s] = from_f32<OT>(p[e]);
                    if (j < i) sAn[t * L::LDC + s] = from_f32<OT>(-a[e]);
                }
                if (j == i) {
                    // T_ii = (I + A_ii)^{-1}, in registers (accumulator layout)
                    const f32x4 tinv = unit_lower_inverse16(a);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sTd[(16 * i + 4 * gq + e) * L::LDD + r16] = from_f32<OT>(tinv[e]);
                }
            }
        }

        // ---- K+ S and Q+ S (registers only; independent of the Gram work) ----
        f32x4 KS[4], QS[4];
        if constexpr (!CH) {
            Frag<OT> Sb[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) Sb[kb] = reg_frag<OT>(S_acc[2 * kb], S_acc[2 * kb + 1]);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = ak;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    ak = mma(ak, lds_frag(sK, L::LDK, 16 * rt, 32 * kb), Sb[kb]);
                    aq = mma(aq, lds_frag(sQ, L::LDK, 16 * rt, 32 * kb), Sb[kb]);
                }
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(wEg + 16 * rt + 4 * gq);
                KS[rt] = ak * eg;
                QS[rt] = aq * eg;
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                // rows of block rt read S scaled by e^{R_rt} per key channel
                f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = ak;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const f32x4 e0 = *reinterpret_cast<const f32x4 *>(sER + rt * K + 32 * kb + 4 * gq);
                    const f32x4 e1 = *reinterpret_cast<const f32x4 *>(sER + rt * K + 32 * kb + 16 + 4 * gq);
                    const Frag<OT> sb = reg_frag<OT>(S_acc[2 * kb] * e0, S_acc[2 * kb + 1] * e1);
                    ak = mma(ak, lds_frag(sK, L::LDK, 16 * rt, 32 * kb), sb);
                    aq = mma(aq, lds_frag(sQ, L::LDK, 16 * rt, 32 * kb), sb);
                }
                KS[rt] = ak;
                QS[rt] = aq;
            }
        }
        lds_barrier();   // -A blocks, P and T_ii of all waves are visible

        // ---- state chain (per wave, its 16 value columns) ----
        {
            // X = diag(beta) (V - K+ S); with decoupled gates
            // X = diag(w) V - diag(e) K+ S (e in beta's place)
            f32x4 X[4];
            const bool dgate = args.wgate != nullptr;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const f32x4 bt = *reinterpret_cast<const f32x4 *>(sBeta + 16 * rt + 4 * gq);
                const f32x4 wt = *reinterpret_cast<const f32x4 *>(sWg + 16 * rt + 4 * gq);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 16 * rt + 4 * gq + e;
                    const float vv = to_f32(sV[t * L::LDC + vcol]);
                    X[rt][e] = dgate ? wt[e] * vv - bt[e] * KS[rt][e] : bt[e] * (vv - KS[rt][e]);
                }
            }
            // (I + A) D = X by block forward substitution (sAn holds -A)
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 D[4];
            D[0] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 0, 0), reg_frag<OT>(X[0], z));
            f32x4 Y = mma_lo(X[1], lds_frag_lo(sAn, L::LDC, 16, 0), reg_frag<OT>(D[0], z));
            D[1] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 16, 0), reg_frag<OT>(Y, z));
            const Frag<OT> Df0 = reg_frag<OT>(D[0], D[1]);
            Y = mma(X[2], lds_frag(sAn, L::LDC, 32, 0), Df0);
            f32x4 Y3 = mma(X[3], lds_frag(sAn, L::LDC, 48, 0), Df0);
            D[2] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 32, 0), reg_frag<OT>(Y, z));
            Y3 = mma_lo(Y3, lds_frag_lo(sAn, L::LDC, 48, 32), reg_frag<OT>(D[2], z));
            D[3] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 48, 0), reg_frag<OT>(Y3, z));
            const Frag<OT> Df1 = reg_frag<OT>(D[2], D[3]);

            // O = Q+ S + P D, staged in sO for 16-byte stores
            f32x4 O[4];
            O[0] = mma_lo(QS[0], lds_frag_lo(sP, L::LDC, 0, 0), Df0);
            O[1] = mma(QS[1], lds_frag(sP, L::LDC, 16, 0), Df0);
            O[2] = mma(QS[2], lds_frag(sP, L::LDC, 32, 0), Df0);
            O[2] = mma_lo(O[2], lds_frag_lo(sP, L::LDC, 32, 32), Df1);
            O[3] = mma(QS[3], lds_frag(sP, L::LDC, 48, 0), Df0);
            O[3] = mma(O[3], lds_frag(sP, L::LDC, 48, 32), Df1);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sO[(16 * rt + 4 * gq + e) * L::LDC + vcol] = from_f32<DT>(O[rt][e]);

            // S' = Diag(e^{gamma_n}) S + K-^T D
            Frag<OT> Ef0, Ef1;
            if constexpr (!CH) {
                f32x4 Dt[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    Dt[rt] = D[rt] * *reinterpret_cast<const f32x4 *>(wEgn + 16 * rt + 4 * gq);
                Ef0 = reg_frag<OT>(Dt[0], Dt[1]);
                Ef1 = reg_frag<OT>(Dt[2], Dt[3]);
#pragma unroll
                for (int ct = 0; ct < NT; ++ct) S_acc[ct] *= egN;
            } else {
                Ef0 = Df0;
                Ef1 = Df1;
#pragma unroll
                for (int ct = 0; ct < NT; ++ct)
                    S_acc[ct] *= *reinterpret_cast<const f32x4 *>(sER + 4 * K + 16 * ct + 4 * gq);
            }
#pragma unroll
            for (int ct = 0; ct < NT; ++ct) {
                S_acc[ct] = mma(S_acc[ct], lds_frag_kmt<EPV>(sKmT, L::LDC, 16 * ct, 0), Ef0);
                S_acc[ct] = mma(S_acc[ct], lds_frag_kmt<EPV>(sKmT, L::LDC, 16 * ct, 32), Ef1);
            }
        }
        lds_barrier();
    }
    if (nchunks > 0) flush_o((nchunks - 1) * CH_T, T - (nchunks - 1) * CH_T);

    if (args.S_T) {
        float *ST = args.S_T + (long)bh * K * V;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) ST[(16 * ct + 4 * gq + e) * V + v0 + vcol] = S_acc[ct][e];
    }

    if constexpr (PRO) {
        // The carried states after the sequence: the last three raw tokens (older
        // ones from the incoming state when T < 3).  q and k by the first column
        // block of the head, v by every block for its columns.
        auto state_out = [&](const DT *raw, const DT *cs, void *outp, int E, int c0, int n) {
            DT *out = static_cast<DT *>(outp);
            if (!out) return;
            for (int i = tid; i < 3 * n; i += NTHR) {
                const int r = i / n, c = c0 + i % n, t = T - 3 + r;
                DT x = from_f32<DT>(0.f);
                if (t >= 0) x = raw[(row_base + (long)t * H) * E + c];
                else if (cs) x = cs[((long)b * 3 + 3 + t) * H * E + (long)h * E + c];
                out[((long)b * 3 + r) * H * E + (long)h * E + c] = x;
            }
        };
        if (vb == 0) {
            state_out(qg, csq, args.cs_q_out, K, 0, K);
            state_out(kg, csk, args.cs_k_out, K, 0, K);
        }
        state_out(vg, csv, args.cs_v_out, V, v0, VBLK);
    }
}

template <typename DT, int K, bool CH, bool PRO = false>
static hipError_t launch_chunk(const ChunkArgs &a, hipStream_t stream)
{
    using L = Smem<DT, K, CH, PRO>;
    static bool attr_set = false;  // benign race: every thread sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_fwd_kernel<DT, K, CH, PRO>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const long nwg = (long)a.B * a.H * a.nvb;
    hipLaunchKernelGGL((chunk_fwd_kernel<DT, K, CH, PRO>), dim3((unsigned)nwg), dim3(NTHR), L::bytes,
                       stream, a);
    return hipGetLastError();
}

hipError_t chunk_fwd_ws_launch(int K, const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *S0, void *o, float *S_T, int B,
                               int T, int H, int V, hipStream_t st);
hipError_t chunk_fwd_wsc_launch(int K, const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *S0, void *o, float *S_T, int B,
                                int T, int H, int V, hipStream_t st);
hipError_t chunk_fwd_wsc_dg_launch(int K, const void *q, const void *k, const void *v, const float *g,
                                   const float *erase, const float *write, const float *S0, void *o,
                                   float *S_T, int B, int T, int H, int V, hipStream_t st);
hipError_t chunk_fwd_ws_dg_launch(int K, const void *q, const void *k, const void *v, const float *g,
                                  const float *erase, const float *write, const float *S0, void *o,
                                  float *S_T, int B, int T, int H, int V, hipStream_t st);

static ChunkArgs chunk_args(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *wgate, const float *S0, void *o,
                            float *S_T, int B, int T, int H, int V)
{
    ChunkArgs a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S0 = S0; a.o = o; a.S_T = S_T;
    a.wgate = wgate;
    a.B = B; a.T = T; a.H = H; a.V = V;
    a.nvb = V / VBLK;
    const long bhn = (long)B * H;
    // The hardware hands consecutive workgroups to the 8 XCDs in turn; keep the
    // column blocks of one head on one XCD so its q/k/g are fetched into one L2.
    a.xcd_map = (a.nvb > 1 && bhn % 8 == 0) ? 1 : 0;
    return a;
}

// Host entry used by the C ABI after validation.  bf16 operands take the
// warp-specialised kernels (chunk_fwd_ws.hip for the scalar gate,
// chunk_fwd_wsc.hip for the per-channel gate).
hipError_t chunk_fwd_launch(bool bf16, bool channel, int K, const void *q, const void *k,
                            const void *v, const float *g, const float *beta, const float *S0,
                            void *o, float *S_T, int B, int T, int H, int V, hipStream_t st)
{
    if (bf16 && !channel)
        return chunk_fwd_ws_launch(K, q, k, v, g, beta, S0, o, S_T, B, T, H, V, st);
    if (bf16 && channel)
        return chunk_fwd_wsc_launch(K, q, k, v, g, beta, S0, o, S_T, B, T, H, V, st);
    const ChunkArgs a = chunk_args(q, k, v, g, beta, nullptr, S0, o, S_T, B, T, H, V);
    // fp32 operands (K = 64)
    return channel ? launch_chunk<float, 64, true>(a, st) : launch_chunk<float, 64, false>(a, st);
}

// Decoupled erase/write gates (erase in beta's place, write gate w): bf16
// takes the warp-specialised kernels' decoupled instantiations; fp32 the
// kernel above.
hipError_t chunk_fwd_dg_launch(bool bf16, bool channel, int K, const void *q, const void *k,
                               const void *v, const float *g, const float *erase,
                               const float *write, const float *S0, void *o, float *S_T, int B,
                               int T, int H, int V, hipStream_t st)
{
    if (bf16 && channel)
        return chunk_fwd_wsc_dg_launch(K, q, k, v, g, erase, write, S0, o, S_T, B, T, H, V, st);
    if (bf16)
        return chunk_fwd_ws_dg_launch(K, q, k, v, g, erase, write, S0, o, S_T, B, T, H, V, st);
    const ChunkArgs a = chunk_args(q, k, v, g, erase, write, S0, o, S_T, B, T, H, V);
    if (!bf16)
        return channel ? launch_chunk<float, 64, true>(a, st) : launch_chunk<float, 64, false>(a, st);
    if (K == 64)
        return channel ? launch_chunk<__bf16, 64, true>(a, st) : launch_chunk<__bf16, 64, false>(a, st);
    return channel ? launch_chunk<__bf16, 128, true>(a, st) : launch_chunk<__bf16, 128, false>(a, st);
}

} // namespace gdn

namespace gdn {

// The prologue fused into the chunk kernel (raw projections in, o and S_T out):
// every storage type, gate and K (fp32: K = 64).  p carries the raw inputs, the
// taps, the carried states and the cap in the prologue's own layout.
hipError_t chunk_fwd_pro_launch(bool bf16, bool channel, bool silu, int K, const PrArgs &p,
                                const float *S0, void *o, float *S_T, int V, hipStream_t st)
{
    ChunkArgs a = chunk_args(p.q_raw, p.k_raw, p.v_raw, p.g_raw, p.b_raw, nullptr, S0, o, S_T,
                             p.B, p.T, p.H, V);
    a.w_q = p.w_q; a.w_k = p.w_k; a.w_v = p.w_v;
    a.cs_q = p.cs_q; a.cs_k = p.cs_k; a.cs_v = p.cs_v;
    a.cs_q_out = p.cs_q_out; a.cs_k_out = p.cs_k_out; a.cs_v_out = p.cs_v_out;
    a.cap = p.cap;
    a.silu = silu ? 1 : 0;
    if (!bf16)
        return channel ? launch_chunk<float, 64, true, true>(a, st)
                       : launch_chunk<float, 64, false, true>(a, st);
    if (K == 64)
        return channel ? launch_chunk<__bf16, 64, true, true>(a, st)
                       : launch_chunk<__bf16, 64, false, true>(a, st);
    return channel ? launch_chunk<__bf16, 128, true, true>(a, st)
                   : launch_chunk<__bf16, 128, false, true>(a, st);
}

} // namespace gdn
