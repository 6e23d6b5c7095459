// chunk_fwd_wsc.hip -- warp-specialised chunkwise forward for bf16 operands and
// the per-key-channel gate (GDN-2 / KDA: one log-decay per key channel).
//
// Mathematics (Atomic-GDN2 model card, section 2.1; the chunkwise mode of the
// MindPattern "Gated DeltaNet" page).  For a chunk of 64 tokens in four blocks
// of 16, with g in [-5, 0] per token and key channel c:
//   lambda_tc  running sum of g_c from the start of t's block (|lambda| <= 80)
//   E_bc       e^{sum of g_c over block b}                   (<= 1)
//   R_ic       sum of g_c over the blocks before i,  gn_c the chunk total
//   KL = k e^{lambda},  QL = q e^{lambda},  KI = k e^{-lambda}  (<= e^80: fits bf16)
//   K+ S (rows of block i) = KL_i (Diag(e^{R_i}) S),  likewise Q+ S with QL_i
//   A_ij = diag(beta_i) KL_i (KI_j * F_ij)^T,  P_ij = QL_i (KI_j * F_ij)^T,
//          F_ij = e^{R_i - R_j} = E_j ... E_{i-1} per channel (1 for i = j)
//   (I + A) D = diag(beta)(V - K+ S),  O = Q+ S + P D,
//   S' = Diag(e^{gn}) S + K-^T D,  K- = KI e^{gn - R_i}  (<= 1).
// Every exponential stays in range because the decay is split at 16-token
// blocks (the card notes that its kernel bounds the decay for the same reason).
//
// Work split (as in chunk_fwd_ws.hip): 4 chain waves own 16 value columns each
// of the fp32 state and run chunk c; 4 prep waves get chunk c+1 ready.  Prep
// wave w owns token block w of the chunk: it loads that block's q, k, g (the
// MFMA fragment layout, straight from global memory), scans g across its 16
// rows with DPP, forms KL, QL, KI and writes them to LDS; after the prep waves
// have met (all block totals E written), they write the chain factors (one
// channel per lane) and each scales its KI into K-.  The Gram blocks (diagonal
// blocks with their inverses, and the six off-diagonal blocks) are left to the
// chain waves, which are idle once their state update for chunk c is done;
// they start as soon as the prep waves have met.  The chain waves take v straight from global memory one
// chunk ahead and write O straight from their accumulators.
#include "ws_common.h"
#include <type_traits>

namespace gdn {

constexpr int WC_T = 64;       // tokens per chunk
constexpr int WC_VB = 64;      // value columns per workgroup
constexpr int WC_NTHR = 512;   // 4 chain waves + 4 prep waves

// DEC: decoupled erase/write gates (the derived buffer also holds w_t).
template <int K, bool DEC = false> struct WcSmem {
    static constexpr int al(int x) { return (x + 255) & ~255; }
    static constexpr int RB = K * 2;              // bytes per tile row
    static constexpr int CPR = RB / 16;           // 16-byte chunks per row
    static constexpr int TILE = WC_T * RB;
    static constexpr int PAD = 8;
    static constexpr int LDC = WC_T + PAD;        // rows of -A and P (fragment order)
    static constexpr int LDD = 16;                // rows of T_ii
    // chain buffers (two): KL, QL, K- of a chunk, row-major, chunks swizzled
    static constexpr int cKL = 0, cQL = TILE, cKM = 2 * TILE;
    static constexpr int CBUF = 3 * TILE;
    static constexpr int oC = 0;
    // KI of the chunk being prepared (the A operands of the Gram blocks)
    static constexpr int oKI = oC + 2 * CBUF;
    static constexpr int oD = oKI + TILE;
    // derived buffers (two)
    static constexpr int dAn = 0;                           // [48][LDC] rows 16..63 of -A
    static constexpr int dP = dAn + (WC_T - 16) * LDC * 2;  // [64][LDC] P
    static constexpr int dTd = dP + WC_T * LDC * 2;         // [64][16] T_ii
    static constexpr int dBeta = dTd + WC_T * LDD * 2;      // beta_t (decoupled gates: e_t)
    static constexpr int dW = dBeta + WC_T * 4;             // decoupled gates: w_t
    static constexpr int dCF = dW + (DEC ? WC_T * 4 : 0);   // [4][K]: e^{R_1}, e^{R_2}, e^{R_3}, e^{gn}
    static constexpr int DBUF = al(dCF + 4 * K * 4);
    static constexpr int kE = oD + 2 * DBUF;                // [4][K] E_b of the chunk being prepared
    static constexpr int kAd = kE + 4 * K * 4;              // [4][16][16] fp32 -A of diagonal blocks
    static constexpr int kCtr = kAd + 4 * 16 * 16 * 4;
    static constexpr int bytes = al(kCtr + 16);
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Byte offset of the 16-byte chunk `ch` of row `row` of a q/k-shaped tile
// (rows of CPR chunks).  For 128 keys the chunk index is XORed with the row's
// low four bits in swapped halves, so that both the 16-row fragment reads (one
// chunk of 16 consecutive rows) and the transposed reads (four chunks of four
// consecutive rows) fall on distinct banks; 64 keys use the plain row XOR.
template <int CPR> __device__ __forceinline__ int wc_off(int row, int ch) {
    if constexpr (CPR == 16)
        return row * 256 + ((ch ^ (((row & 3) << 2) | ((row >> 2) & 3))) << 4);
    else
        return qk_off<CPR>(row, ch);
}
// Fragment: rows row0 + r16, keys 32 kb + 8 gq .. +7 (one 16-byte read).
template <int CPR> __device__ __forceinline__ Frag<__bf16> wc_frag(const char *M, int row0, int kb) {
    return {*reinterpret_cast<const bf16x8 *>(M + wc_off<CPR>(row0 + lane_r16(), 4 * kb + lane_gq()))};
}

// 8 bf16 scaled by 8 factors (fp32 arithmetic), back to bf16.
__device__ __forceinline__ bf16x8 scale8(bf16x8 x, f32x4 f0, f32x4 f1) {
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (float)x[e] * f0[e];
        b[e] = (float)x[4 + e] * f1[e];
    }
    return cat8(cvt4(a), cvt4(b));
}

struct WcArgs {
    const __bf16 *q, *k, *v;
    const float *g, *beta, *S0;
    __bf16 *o;
    float *S_T;
    int T, H, V, nvb;
    int xcd_map;
    // Segments (seg_len > 0): workgroup w runs chunks [seg seg_len, (seg + 1)
    // seg_len) of its (b, h, column block), seg = w / nbhv, starting from S0 for
    // segment 0 and from Sb[b h][seg - 1] ([B*H][nseg-1][K][V] fp32) after it.
    int seg_len, nseg;
    long nbhv;
    const float *Sb;
    // Decoupled erase/write gates (reading of the MindPattern "Gated DeltaNet"
    // page, finding of 2026-05-22): beta carries the erase gate e and wgate the
    // write gate w; only the DEC instantiations read it.
    const float *wgate;
};

// WO = false: the final state only (no o).  q is then not read, and QL, P, Q+ S
// and O are not formed: the state update needs none of them.
// DEC = true: decoupled gates, S_t = (I - e_t k k^T) Diag(alpha_t) S + w_t k v^T.
// The chunk algebra is the same with e in beta's place in (I + A) and on the
// right side X = diag(w) V - diag(e) K+ S.
template <int K, bool WO, bool DEC>
__global__ __launch_bounds__(WC_NTHR, 1) void chunk_fwd_wsc_kernel(WcArgs args)
{
    using L = WcSmem<K, DEC>;
    constexpr int NT = K / 16;          // 16-row tiles of S
    constexpr int NKB = K / 32;         // 32-key blocks
    constexpr int CPR = L::CPR;

    extern __shared__ __attribute__((aligned(256))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int gq = lane >> 4;

    const int T = args.T, H = args.H, V = args.V, nvb = args.nvb;
    int bh, vb, seg = 0;
    {
        int w = blockIdx.x;
        if (args.seg_len > 0) {
            seg = (int)(w / args.nbhv);
            w = (int)(w % args.nbhv);
        }
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
    const int v0 = vb * WC_VB;
    const long row_base = (long)b * T * H + h;   // row of token 0 in [B*T*H]
    const int nch_all = (T + WC_T - 1) / WC_T;
    const int c0 = args.seg_len > 0 ? seg * args.seg_len : 0;                    // first chunk
    const int c1 = args.seg_len > 0 ? min(nch_all, c0 + args.seg_len) : nch_all; // end

    auto cbuf = [&](int c) { return smem + L::oC + (c & 1) * L::CBUF; };
    auto dbuf = [&](int c) { return smem + L::oD + (c & 1) * L::DBUF; };
    char *sKI = smem + L::oKI;
    float *sE = reinterpret_cast<float *>(smem + L::kE);
    unsigned *ctr = reinterpret_cast<unsigned *>(smem + L::kCtr);
    if (tid == 0) *ctr = 0u;
    lds_barrier();

    if (wave >= 4) {
        // ============================ prep waves ============================
        const int pw = __builtin_amdgcn_readfirstlane(wave - 4);   // token block of this wave
        const int row = 16 * pw + r16;                             // token row of this lane
        // raw q, k, g of this lane's row, fragment layout: keys 32 kb + 8 gq .. +7
        bf16x8 rk[NKB], rq[NKB];
        f32x4 rg[NKB][2];
        float rb = 0.f, rw = 0.f;
        // Loads of one key block (k, q, g) or of beta for chunk n; rows past T
        // read as zero (g = beta = 0: they change nothing).
        auto fetch_kb = [&](int n, int kb) __attribute__((always_inline)) {
            const int t = n * WC_T + row;
            if (t < T) {
                const long off = (row_base + (long)t * H) * K + 32 * kb + 8 * gq;
                rk[kb] = *reinterpret_cast<const bf16x8 *>(args.k + off);
                if constexpr (WO) rq[kb] = *reinterpret_cast<const bf16x8 *>(args.q + off);
                rg[kb][0] = *reinterpret_cast<const f32x4 *>(args.g + off);
                rg[kb][1] = *reinterpret_cast<const f32x4 *>(args.g + off + 4);
            } else {
                rk[kb] = bf16x8{};
                if constexpr (WO) rq[kb] = bf16x8{};
                rg[kb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                rg[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        auto fetch_beta = [&](int n) __attribute__((always_inline)) {
            const int t = n * WC_T + row;
            rb = t < T ? args.beta[row_base + (long)t * H] : 0.f;
            if constexpr (DEC) rw = t < T ? args.wgate[row_base + (long)t * H] : 0.f;
        };

        unsigned arrivals = 0;
        auto prepare = [&](int n) __attribute__((always_inline)) {
            char *C = cbuf(n);
            char *D = dbuf(n);
            float *sCF = reinterpret_cast<float *>(D + L::dCF);

            // --- this block's rows: lambda, E_pw, KL, QL, KI (kept), beta
            // lambda: each scan step over all 32 values of the lane at once, so the
            // dependent DPP adds of one value interleave with the others
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = rg[kb][hh][e];
                            rg[kb][hh][e] = x + (st == 0 ? dpp_shr<0x111>(x) : st == 1 ? dpp_shr<0x112>(x)
                                                 : st == 2 ? dpp_shr<0x114>(x) : dpp_shr<0x118>(x));
                        }
            Frag<__bf16> fKL[NKB], fQL[NKB], fKI[NKB];   // KI kept for K-
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                f32x4 el[2], ei[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // lambda log2(e), then e^{lambda} and e^{-lambda} by exp2
                        const float x = rg[kb][hh][e] * 1.44269504088896341f;
                        el[hh][e] = __builtin_amdgcn_exp2f(x);
                        ei[hh][e] = __builtin_amdgcn_exp2f(-x);
                    }
                fKL[kb].v = scale8(rk[kb], el[0], el[1]);
                if constexpr (WO) fQL[kb].v = scale8(rq[kb], el[0], el[1]);
                fKI[kb].v = scale8(rk[kb], ei[0], ei[1]);
                // this key block of the next chunk goes in flight (spread over the
                // loop rather than issued as one burst)
                if (n + 1 < c1) fetch_kb(n + 1, kb);
                const int off = wc_off<CPR>(row, 4 * kb + gq);
                *reinterpret_cast<bf16x8 *>(C + L::cKL + off) = fKL[kb].v;
                if constexpr (WO) *reinterpret_cast<bf16x8 *>(C + L::cQL + off) = fQL[kb].v;
                *reinterpret_cast<bf16x8 *>(sKI + off) = fKI[kb].v;
                if (r16 == 15) {   // block totals: E_pw = e^{lambda of the last row}
                    float *eb = sE + pw * K + 32 * kb + 8 * gq;
                    *reinterpret_cast<f32x4 *>(eb) = el[0];
                    *reinterpret_cast<f32x4 *>(eb + 4) = el[1];
                }
            }
            if (gq == 0) {
                reinterpret_cast<float *>(D + L::dBeta)[row] = rb;
                if constexpr (DEC) reinterpret_cast<float *>(D + L::dW)[row] = rw;
            }
            if (n + 1 < c1) fetch_beta(n + 1);
            arrivals += 4;
            prep_barrier(ctr, arrivals);         // KL, QL, KI and E of all blocks written

            // --- chain factors e^{R_1} = E_0, e^{R_2}, e^{R_3}, e^{gn}: one channel
            //     per lane (wave w takes channels w K/4 .. (w+1) K/4 - 1)
            if (lane < K / 4) {
                const int c = (K / 4) * pw + lane;
                const float e0 = sE[c], e1 = sE[K + c], e2 = sE[2 * K + c], e3 = sE[3 * K + c];
                const float e01 = e0 * e1, e012 = e01 * e2;
                sCF[c] = e0;
                sCF[K + c] = e01;
                sCF[2 * K + c] = e012;
                sCF[3 * K + c] = e012 * e3;
            }
            // --- K- of this block: KI * e^{gn - R_pw} = KI * E_pw ... E_3 (all
            //     factors read before any tile write)
            auto kminus = [&](auto pwc) __attribute__((always_inline)) {
                constexpr int PW = decltype(pwc)::value;
                bf16x8 km[NKB];
#pragma unroll
                for (int hb = 0; hb < NKB; hb += NKB / 2) {
                    f32x4 E[NKB / 2][4 - PW][2];
#pragma unroll
                    for (int i = 0; i < NKB / 2; ++i)
#pragma unroll
                        for (int bb = PW; bb < 4; ++bb) {
                            const float *F = sE + bb * K + 32 * (hb + i) + 8 * gq;
                            E[i][bb - PW][0] = *reinterpret_cast<const f32x4 *>(F);
                            E[i][bb - PW][1] = *reinterpret_cast<const f32x4 *>(F + 4);
                        }
                    GDN_SCHED_FENCE();
#pragma unroll
                    for (int i = 0; i < NKB / 2; ++i) {
                        f32x4 f0 = E[i][0][0], f1 = E[i][0][1];
#pragma unroll
                        for (int bb = PW + 1; bb < 4; ++bb) {
                            f0 *= E[i][bb - PW][0];
                            f1 *= E[i][bb - PW][1];
                        }
                        km[hb + i] = scale8(fKI[hb + i].v, f0, f1);
                    }
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    *reinterpret_cast<bf16x8 *>(C + L::cKM + wc_off<CPR>(row, 4 * kb + gq)) = km[kb];
            };
            if (pw == 0) kminus(std::integral_constant<int, 0>());
            else if (pw == 1) kminus(std::integral_constant<int, 1>());
            else if (pw == 2) kminus(std::integral_constant<int, 2>());
            else kminus(std::integral_constant<int, 3>());
        };

        if (c0 < c1) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) fetch_kb(c0, kb);
            fetch_beta(c0);
            prepare(c0);
            lds_barrier();
        }
        for (int c = c0; c < c1; ++c) {
            if (c + 1 < c1) prepare(c + 1);
            lds_barrier();
        }
        return;
    }

    // ============================= chain waves =============================
    // Accumulator tile ct = 2kb + hh, lane (gq, r16), element e holds S[key][col]
    // with key = 32kb + 8gq + 4hh + e and col = v0 + 16 wave + r16.
    const int vcol = 16 * wave + r16;
    auto key_of = [&](int ct, int e) { return 32 * (ct >> 1) + 8 * gq + 4 * (ct & 1) + e; };
    f32x4 S_acc[NT];
    {
        const float *S0 = seg > 0 ? args.Sb + ((long)bh * (args.nseg - 1) + seg - 1) * K * V
                        : args.S0 ? args.S0 + (long)bh * K * V : nullptr;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S_acc[ct][e] = S0 ? S0[key_of(ct, e) * V + v0 + vcol] : 0.f;
    }
    // v of a chunk in the accumulator layout (rows 16 rt + 4 gq + e of this
    // lane's column), loaded one chunk ahead; rows past T repeat row T-1
    const unsigned v_lane = (unsigned)(4 * gq * H * V + v0 + vcol);   // row 4 gq of a chunk
    unsigned short vr[4][4];
    const unsigned short *vsrc = reinterpret_cast<const unsigned short *>(args.v);
    auto fetch_v = [&](int n) __attribute__((always_inline)) {
        if ((n + 1) * WC_T <= T) {
            // whole chunk inside the sequence: a wave-uniform base per row (scalar
            // address arithmetic) and one 32-bit lane offset
            const unsigned short *pn = vsrc + (row_base + (long)n * WC_T * H) * V;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) vr[rt][e] = (pn + (long)(16 * rt + e) * H * V)[v_lane];
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = min(n * WC_T + 16 * rt + 4 * gq + e, T - 1);
                    vr[rt][e] = vsrc[(row_base + (long)t * H) * V + v0 + vcol];
                }
        }
    };
    float *sAd = reinterpret_cast<float *>(smem + L::kAd) + wave * 256;   // -A of a diagonal block
    // Gram blocks of chunk n, once the prep waves have written KL, QL, KI, E
    // and beta: the diagonal block of this wave's index and its inverse T_ii,
    // then off-diagonal blocks (I, J): A = KI_J * F_IJ (per channel),
    // B = KL_I and QL_I, computed transposed (the product's rows are s of block
    // J, its columns t of block I), so that each lane holds four consecutive
    // columns s of one row t:
    //   w0: (1,0) (3,0)   w1: (2,1) (3,1)   w2: (3,2)   w3: (2,0)
    // F_IJ = E_J ... E_{I-1} per channel.
    auto gram_pairs = [&](int n) __attribute__((always_inline)) {
        wait_arrivals(ctr, 4u * (unsigned)(n - c0 + 1));   // prepare(c0 .. n) arrived
        const char *C = cbuf(n);
        char *D = dbuf(n);
        __bf16 *sAn = reinterpret_cast<__bf16 *>(D + L::dAn);
        __bf16 *sP = reinterpret_cast<__bf16 *>(D + L::dP);
        const float *sBn = reinterpret_cast<const float *>(D + L::dBeta);
        // Blocks (I1, J) and, if I2 > 0, (I2, J) (they share the A source KI_J),
        // half of the key blocks at a time: every LDS read of the half is issued
        // before any product.
        auto pairs = [&](auto i1c, auto i2c, auto jc) __attribute__((always_inline)) {
            constexpr int I1 = decltype(i1c)::value, I2 = decltype(i2c)::value, J = decltype(jc)::value;
            constexpr int IM = I2 > 0 ? I2 : I1;       // E rows J .. IM-1 are needed
            constexpr int NH = NKB / 2;
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 aA1 = z, aP1 = z, aA2 = z, aP2 = z;
#pragma unroll
            for (int hb = 0; hb < NKB; hb += NH) {
                Frag<__bf16> fa[NH], fk1[NH], fq1[NH], fk2[NH], fq2[NH];
                f32x4 E[NH][IM - J][2];
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const int kb = hb + i;
                    fa[i] = wc_frag<CPR>(sKI, 16 * J, kb);
                    fk1[i] = wc_frag<CPR>(C + L::cKL, 16 * I1, kb);
                    if constexpr (WO) fq1[i] = wc_frag<CPR>(C + L::cQL, 16 * I1, kb);
                    if constexpr (I2 > 0) {
                        fk2[i] = wc_frag<CPR>(C + L::cKL, 16 * I2, kb);
                        if constexpr (WO) fq2[i] = wc_frag<CPR>(C + L::cQL, 16 * I2, kb);
                    }
#pragma unroll
                    for (int bb = J; bb < IM; ++bb) {
                        const float *F = sE + bb * K + 32 * kb + 8 * gq;
                        E[i][bb - J][0] = *reinterpret_cast<const f32x4 *>(F);
                        E[i][bb - J][1] = *reinterpret_cast<const f32x4 *>(F + 4);
                    }
                }
                GDN_SCHED_FENCE();
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    f32x4 f0 = E[i][0][0], f1 = E[i][0][1];
#pragma unroll
                    for (int bb = J + 1; bb < I1; ++bb) {
                        f0 *= E[i][bb - J][0];
                        f1 *= E[i][bb - J][1];
                    }
                    const Frag<__bf16> a1 = {scale8(fa[i].v, f0, f1)};
                    aA1 = mma(aA1, a1, fk1[i]);
                    if constexpr (WO) aP1 = mma(aP1, a1, fq1[i]);
                    if constexpr (I2 > 0) {
#pragma unroll
                        for (int bb = I1; bb < I2; ++bb) {
                            f0 *= E[i][bb - J][0];
                            f1 *= E[i][bb - J][1];
                        }
                        const Frag<__bf16> a2 = {scale8(fa[i].v, f0, f1)};
                        aA2 = mma(aA2, a2, fk2[i]);
                        if constexpr (WO) aP2 = mma(aP2, a2, fq2[i]);
                    }
                }
            }
            const int s0 = 16 * J + 4 * gq;
            {
                const int t = 16 * I1 + r16;
                *reinterpret_cast<bf16x4 *>(sAn + (t - 16) * L::LDC + frag_col(s0)) = cvt4(aA1 * -sBn[t]);
                if constexpr (WO) *reinterpret_cast<bf16x4 *>(sP + t * L::LDC + frag_col(s0)) = cvt4(aP1);
            }
            if constexpr (I2 > 0) {
                const int t = 16 * I2 + r16;
                *reinterpret_cast<bf16x4 *>(sAn + (t - 16) * L::LDC + frag_col(s0)) = cvt4(aA2 * -sBn[t]);
                if constexpr (WO) *reinterpret_cast<bf16x4 *>(sP + t * L::LDC + frag_col(s0)) = cvt4(aP2);
            }
        };
        using std::integral_constant;
        const int cw = __builtin_amdgcn_readfirstlane(wave);
        // diagonal block cw (F = 1, masked) and its inverse
        {
            f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = aA;
            Frag<__bf16> fi[NKB], fl[NKB], fq[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                fi[kb] = wc_frag<CPR>(sKI, 16 * cw, kb);
                fl[kb] = wc_frag<CPR>(C + L::cKL, 16 * cw, kb);
                if constexpr (WO) fq[kb] = wc_frag<CPR>(C + L::cQL, 16 * cw, kb);
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                aA = mma(aA, fi[kb], fl[kb]);
                if constexpr (WO) aP = mma(aP, fi[kb], fq[kb]);
            }
            const int t = 16 * cw + r16, s0 = 16 * cw + 4 * gq;
            const float bt = sBn[t];
            f32x4 a, p;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = s0 + e;
                a[e] = (s < t) ? bt * aA[e] : 0.f;
                p[e] = (s <= t) ? aP[e] : 0.f;
            }
            if constexpr (WO) *reinterpret_cast<bf16x4 *>(sP + t * L::LDC + frag_col(s0)) = cvt4(p);
            // -A of the block row-major; this wave reads it back, in order, for the inverse
            *reinterpret_cast<f32x4 *>(sAd + r16 * 16 + 4 * gq) = -a;
            const f32x4 tr = unit_lower_inverse16_rows(sAd);
            *reinterpret_cast<bf16x4 *>(reinterpret_cast<__bf16 *>(D + L::dTd) + (16 * cw + (lane >> 2)) * L::LDD +
                                        4 * (lane & 3)) = cvt4(tr);
        }
        if (cw == 0) pairs(integral_constant<int, 1>(), integral_constant<int, 3>(), integral_constant<int, 0>());
        else if (cw == 1) pairs(integral_constant<int, 2>(), integral_constant<int, 3>(), integral_constant<int, 1>());
        else if (cw == 2) pairs(integral_constant<int, 3>(), integral_constant<int, 0>(), integral_constant<int, 2>());
        else pairs(integral_constant<int, 2>(), integral_constant<int, 0>(), integral_constant<int, 0>());
    };
    if (c0 < c1) {
        fetch_v(c0);
        gram_pairs(c0);
        lds_barrier();     // chunk c0 is ready
    }

    const int trow = 4 * gq + (r16 >> 2), tq = r16 & 3;
    int k_tr[NKB];                         // + 8 hh + RB (32 kb2 + 16 s)
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) k_tr[kk] = wc_off<CPR>(trow, 4 * kk + tq);

    for (int c = c0; c < c1; ++c) {
        const char *C = cbuf(c);
        const char *sKL = C + L::cKL, *sQL = C + L::cQL, *sKM = C + L::cKM;
        const char *D = dbuf(c);
        const __bf16 *sAn = reinterpret_cast<const __bf16 *>(D + L::dAn);
        const __bf16 *sP = reinterpret_cast<const __bf16 *>(D + L::dP);
        const __bf16 *sTd = reinterpret_cast<const __bf16 *>(D + L::dTd);
        const float *sBeta = reinterpret_cast<const float *>(D + L::dBeta);
        const float *sW = reinterpret_cast<const float *>(D + L::dW);   // decoupled gates only
        const float *sCF = reinterpret_cast<const float *>(D + L::dCF);
        unsigned ktr_addr[NKB];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) ktr_addr[kk] = opaque(lds_u32(sKM) + k_tr[kk]);

        // Phase A: K+ S and Q+ S.  Row tile rt (token block rt) takes the state
        // with its key rows scaled by e^{R_rt}.
        // QS and O are computed transposed (rows: value columns, columns:
        // tokens), by swapping the MFMA operands: the same fragments serve, and
        // each lane ends with four consecutive value columns of one token.
        f32x4 KS[4], QS[4];
        {
            Frag<__bf16> fk[NKB], fq[NKB];
            f32x4 cfv[2][NKB][2];                  // e^{R_rt} of this lane's keys, one tile ahead
            auto load_cf = [&](int rt) __attribute__((always_inline)) {
                const float *cf = sCF + (rt - 1) * K + 8 * gq;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    cfv[rt & 1][kb][0] = *reinterpret_cast<const f32x4 *>(cf + 32 * kb);
                    cfv[rt & 1][kb][1] = *reinterpret_cast<const f32x4 *>(cf + 32 * kb + 4);
                }
            };
            load_cf(1);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (rt >= 1 && rt + 1 < 4) load_cf(rt + 1);
                Frag<__bf16> Sb[NKB];
                if (rt == 0) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) Sb[kb] = reg_frag<__bf16>(S_acc[2 * kb], S_acc[2 * kb + 1]);
                } else {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
                        Sb[kb] = reg_frag<__bf16>(S_acc[2 * kb] * cfv[rt & 1][kb][0], S_acc[2 * kb + 1] * cfv[rt & 1][kb][1]);
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    fk[kb] = wc_frag<CPR>(sKL, 16 * rt, kb);
                    if constexpr (WO) fq[kb] = wc_frag<CPR>(sQL, 16 * rt, kb);
                }
                f32x4 ak = {0.f, 0.f, 0.f, 0.f}, aq = ak;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    ak = mma(ak, fk[kb], Sb[kb]);
                    if constexpr (WO) aq = mma(aq, Sb[kb], fq[kb]);   // transposed: (Q+ S)^T
                }
                KS[rt] = ak;
                QS[rt] = aq;
                GDN_SCHED_FENCE();
            }
        }

        // Phase B: X = diag(beta)(V - K+ S), then (I + A) D = X by block forward
        // substitution (-A stored); the next chunk's v goes in flight.
        f32x4 X[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 bt = *reinterpret_cast<const f32x4 *>(sBeta + 16 * rt + 4 * gq);
            if constexpr (DEC) {   // w v - e K+ S
                const f32x4 wt = *reinterpret_cast<const f32x4 *>(sW + 16 * rt + 4 * gq);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[rt][e] = wt[e] * __builtin_bit_cast(float, (unsigned)vr[rt][e] << 16) - bt[e] * KS[rt][e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[rt][e] = bt[e] * (__builtin_bit_cast(float, (unsigned)vr[rt][e] << 16) - KS[rt][e]);
            }
        }
        if (c + 1 < c1) fetch_v(c + 1);
        const Frag<__bf16> fT0 = lds_frag_lo(sTd, L::LDD, 0, 0), fT1 = lds_frag_lo(sTd, L::LDD, 16, 0);
        const Frag<__bf16> fT2 = lds_frag_lo(sTd, L::LDD, 32, 0), fT3 = lds_frag_lo(sTd, L::LDD, 48, 0);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 Dd[4];
        Dd[0] = mma_lo(z, fT0, reg_frag<__bf16>(X[0], z));
        f32x4 Y = mma_lo(X[1], lds_frag_fo_lo(sAn, L::LDC, 0, 0), reg_frag<__bf16>(Dd[0], z));
        Dd[1] = mma_lo(z, fT1, reg_frag<__bf16>(Y, z));
        const Frag<__bf16> Df0 = reg_frag<__bf16>(Dd[0], Dd[1]);
        Y = mma(X[2], lds_frag_fo(sAn, L::LDC, 16, 0), Df0);
        f32x4 Y3 = mma(X[3], lds_frag_fo(sAn, L::LDC, 32, 0), Df0);
        Dd[2] = mma_lo(z, fT2, reg_frag<__bf16>(Y, z));
        Y3 = mma_lo(Y3, lds_frag_fo_lo(sAn, L::LDC, 32, 32), reg_frag<__bf16>(Dd[2], z));
        Dd[3] = mma_lo(z, fT3, reg_frag<__bf16>(Y3, z));
        const Frag<__bf16> Df1 = reg_frag<__bf16>(Dd[2], Dd[3]);
        GDN_SCHED_FENCE();

        // Phase C: O = Q+ S + P D.
        bf16x4 kt[NT][4];
        auto load_ct = [&](int ct) __attribute__((always_inline)) {
            const unsigned pk = ktr_addr[ct >> 1] + 8 * (ct & 1);
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                kt[ct][2 * kb2] = lds_read_tr(pk + L::RB * 32 * kb2);
                kt[ct][2 * kb2 + 1] = lds_read_tr(pk + L::RB * (32 * kb2 + 16));
            }
        };
        load_ct(0);
        load_ct(1);
        f32x4 egn[NT];                     // e^{gn} of this lane's key rows
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) egn[ct] = *reinterpret_cast<const f32x4 *>(sCF + 3 * K + key_of(ct, 0));
        if constexpr (WO) {
            f32x4 O[4];
            O[0] = mma_lo(QS[0], Df0, lds_frag_fo_lo(sP, L::LDC, 0, 0));
            O[1] = mma(QS[1], Df0, lds_frag_fo(sP, L::LDC, 16, 0));
            O[2] = mma(QS[2], Df0, lds_frag_fo(sP, L::LDC, 32, 0));
            O[2] = mma_lo(O[2], Df1, lds_frag_fo_lo(sP, L::LDC, 32, 32));
            O[3] = mma(QS[3], Df0, lds_frag_fo(sP, L::LDC, 48, 0));
            O[3] = mma(O[3], Df1, lds_frag_fo(sP, L::LDC, 48, 32));
            // lane (gq, r16) holds value columns 16 wave + 4 gq .. +3 of token
            // 16 rt + r16: one 8-byte store per row tile
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int t = c * WC_T + 16 * rt + r16;
                if (t < T)
                    *reinterpret_cast<bf16x4 *>(args.o + (row_base + (long)t * H) * V + v0 + 16 * wave + 4 * gq) =
                        cvt4(O[rt]);
            }
        }
        const Frag<__bf16> Ef[2] = {Df0, Df1};
        GDN_SCHED_FENCE();

        // Phase D: S' = Diag(e^{gn}) S + K-^T D, the k^T fragments read two
        // tiles ahead.
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
            if (ct + 2 < NT) load_ct(ct + 2);
            S_acc[ct] *= egn[ct];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
                S_acc[ct] = mma(S_acc[ct], Frag<__bf16>{cat8(kt[ct][2 * kb2], kt[ct][2 * kb2 + 1])}, Ef[kb2]);
            GDN_SCHED_FENCE();
        }
        if (c + 1 < c1) gram_pairs(c + 1);
        lds_barrier();
    }

    if (args.S_T) {
        float *ST = args.S_T + (long)bh * K * V;
#pragma unroll
        for (int ct = 0; ct < NT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) ST[key_of(ct, e) * V + v0 + vcol] = S_acc[ct][e];
    }
}

template <int K, bool WO, bool DEC = false>
static hipError_t launch_wsc(const WcArgs &a, long nwg, hipStream_t stream)
{
    using L = WcSmem<K, DEC>;
    static bool attr_set = false;  // benign race: every thread sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_fwd_wsc_kernel<K, WO, DEC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((chunk_fwd_wsc_kernel<K, WO, DEC>), dim3((unsigned)nwg), dim3(WC_NTHR), L::bytes, stream, a);
    return hipGetLastError();
}

// Host entry for bf16 operands with the per-key-channel gate (K = 64 or 128).
hipError_t chunk_fwd_wsc_launch(int K, const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *S0, void *o, float *S_T, int B,
                                int T, int H, int V, hipStream_t st)
{
    WcArgs a = {};
    a.q = (const __bf16 *)q; a.k = (const __bf16 *)k; a.v = (const __bf16 *)v;
    a.g = g; a.beta = beta; a.S0 = S0; a.o = (__bf16 *)o; a.S_T = S_T;
    a.T = T; a.H = H; a.V = V;
    a.nvb = V / WC_VB;
    const long bhn = (long)B * H;
    a.xcd_map = (a.nvb > 1 && bhn % 8 == 0) ? 1 : 0;
    const long nwg = bhn * a.nvb;
    if (o)
        return K == 64 ? launch_wsc<64, true>(a, nwg, st) : launch_wsc<128, true>(a, nwg, st);
    return K == 64 ? launch_wsc<64, false>(a, nwg, st) : launch_wsc<128, false>(a, nwg, st);
}

// The same for decoupled erase/write gates (erase in beta's place).
hipError_t chunk_fwd_wsc_dg_launch(int K, const void *q, const void *k, const void *v, const float *g,
                                   const float *erase, const float *write, const float *S0, void *o,
                                   float *S_T, int B, int T, int H, int V, hipStream_t st)
{
    WcArgs a = {};
    a.q = (const __bf16 *)q; a.k = (const __bf16 *)k; a.v = (const __bf16 *)v;
    a.g = g; a.beta = erase; a.wgate = write; a.S0 = S0; a.o = (__bf16 *)o; a.S_T = S_T;
    a.T = T; a.H = H; a.V = V;
    a.nvb = V / WC_VB;
    const long bhn = (long)B * H;
    a.xcd_map = (a.nvb > 1 && bhn % 8 == 0) ? 1 : 0;
    const long nwg = bhn * a.nvb;
    if (o)
        return K == 64 ? launch_wsc<64, true, true>(a, nwg, st) : launch_wsc<128, true, true>(a, nwg, st);
    return K == 64 ? launch_wsc<64, false, true>(a, nwg, st) : launch_wsc<128, false, true>(a, nwg, st);
}

} // namespace gdn

namespace gdn {

// The o pass of the sequence-parallel forward (per-key-channel gate, K = V =
// 128, bf16): every (b, h, column block, segment) at once, each segment from
// its incoming state in Sb (segment 0 from S0); no final state is written.
hipError_t chunk_fwd_wsc_seg_launch(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *S0, const float *Sb, void *o,
                                    int B, int T, int H, int nseg, int seg_len, hipStream_t st)
{
    WcArgs a = {};
    a.q = (const __bf16 *)q; a.k = (const __bf16 *)k; a.v = (const __bf16 *)v;
    a.g = g; a.beta = beta; a.S0 = S0; a.o = (__bf16 *)o; a.S_T = nullptr;
    a.T = T; a.H = H; a.V = 128;
    a.nvb = 128 / WC_VB;
    const long bhn = (long)B * H;
    a.xcd_map = bhn % 8 == 0 ? 1 : 0;
    a.seg_len = seg_len;
    a.nseg = nseg;
    a.nbhv = bhn * a.nvb;
    a.Sb = Sb;
    return launch_wsc<128, true>(a, a.nbhv * nseg, st);
}

} // namespace gdn
