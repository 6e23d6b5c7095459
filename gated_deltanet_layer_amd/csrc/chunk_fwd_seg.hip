// chunk_fwd_seg.hip -- sequence-parallel chunkwise forward for the final state
// only: bf16 operands, the per-key-channel gate, K = V = 128.
//
// Mathematics (Atomic-GDN2 model card, section 2.1, the recurrence; the
// chunkwise mode of the MindPattern "Gated DeltaNet" page).  A chunk maps the
// state affinely, S' = M S + N, and so does any run of chunks; maps compose
// associatively (the card's kernel benchmark, section 5.1, compares against an
// associative scan of the same recurrence).  A long sequence is cut into
// segments of whole chunks that run at the same time:
//
//   segment 0 runs the recurrence from the true S0 and leaves its final state
//   in S_T;  every later segment s runs the same chunk recurrence on the
//   augmented state [N | M] (K x (V + K)), started from [0 | I]: the value
//   columns see the segment's v, the K extra columns see v = 0, so at the end
//   N_s is the state the segment reaches from zero and M_s the matrix that
//   carries any incoming state through it.
//
// A second kernel then walks the segments of each head in order,
// S <- M_s S + N_s, in fp32, and writes S_T.
//
// Per chunk (n <= 64 tokens, per key channel c; block b = 16 tokens):
//   lambda_tc  running sum of g_c from the start of t's block (>= -80 for g >= -5)
//   E_bc       e^{block total}, R_b = sum of the blocks before b, gn = chunk total
//   KL = k e^{lambda}, KI = k e^{-lambda}          (Gram operands, in range)
//   K+ = KL e^{R_b} = k e^{gamma},  K- = KI e^{gn - R_b} = k e^{gn - gamma}  (<= 1)
//   G_ij = KL_i (KI_j F_ij)^T,  F_ij = E_j ... E_{i-1}  (j < i; the Gram without beta)
//   A = diag(beta) G (strictly lower),  T_ii = (I + A_ii)^{-1},  T'_ii = T_ii diag(beta_i)
//   D_i = T'_ii (V_i - K+_i S - sum_{j<i} G_ij D_j)   (block forward substitution of
//         (I + A) D = diag(beta)(V - K+ S): beta moved into T')
//   S' = Diag(e^{gn}) S + K-^T D,   with V = 0 in the columns of M.
//
// Work split: one workgroup of 8 waves per (head, segment).  Prep waves 4..7
// get chunk n + 1 ready while chain waves 0..3 run chunk n.  Prep wave p owns
// key block p (keys 32p .. 32p+31) of all 64 tokens: the running sums, the block
// factors, the tiles K+ and K- and, on the matrix cores, its key block's share
// of every Gram block (each an MFMA over exactly its 32 keys, operands from
// registers); the four shares meet in LDS, and after the prep waves have met (an
// LDS arrival counter) each sums its Gram blocks, one of them a diagonal block it
// also inverts.  Chain wave w owns 64 columns of the augmented state in MFMA
// accumulators for the whole segment: value columns 32w .. 32w+31 and the same
// columns of M (none in segment 0; skipped once they have decayed to exactly
// zero).  One workgroup barrier per chunk hands the
// chunk's data over; the chain's data is double-buffered.
//
// LDS layouts, chosen for the matrix-core operand reads (measured on gfx950: a
// 16-byte read by 64 lanes from one contiguous 1 KB runs at about 2.3 ns per
// instruction per CU; 16 rows of 256 bytes read at one 16-byte chunk each, even
// XOR-swizzled, at about 3.9 ns):
//   K+ and V: "fragment-major": the 16 x 32 operand fragment (token block rt,
//     32-column block kb) is 1 KB, lane l's 16 bytes at l * 16.
//   K-: 64 rows of 256 bytes, 16-byte chunks XOR-swizzled by the row, read with
//     the transposing ds_read_b64_tr_b16 (2.4 ns per instruction).
//   -G blocks: four 1 KB fragments in the substitution's operand order; T':
//     64 rows of 16 bf16.
#include "ws_common.h"
#include <mutex>
#include <type_traits>

namespace gdn {

constexpr int SG_T = 64;        // tokens per chunk
constexpr int SG_K = 128;       // keys = value columns
constexpr int SG_NTHR = 512;    // 4 chain waves + 4 prep waves

constexpr int sg_al(int x) { return (x + 255) & ~255; }

struct SgSmem {
    static constexpr int TILE = SG_T * SG_K * 2;  // one 64 x 128 bf16 tile
    static constexpr int LDD = 16;                // row length of T'
    // prep buffer (one): each prep wave's share of the ten Gram blocks (fp32,
    // accumulator order), beta of the chunk
    static constexpr int pPart = 0, pBeta = 4 * 10 * 1024, pAd = pBeta + SG_T * 4;
    static constexpr int PREP = sg_al(pAd + 4 * 256 * 4);
    // hand-over buffers (two): what the chain reads for one chunk
    static constexpr int hKP = 0, hKM = TILE, hV = 2 * TILE, hAn = 3 * TILE;
    static constexpr int hTd = hAn + 4 * 1024;
    static constexpr int hEgn = hTd + SG_T * LDD * 2;
    static constexpr int HBUF = sg_al(hEgn + SG_K * 4);
    static constexpr int oH = PREP;
    static constexpr int kCtr = oH + 2 * HBUF;
    static constexpr int bytes = sg_al(kCtr + 16);
    static_assert(bytes <= 160 * 1024, "LDS budget");
};

// Byte offset of the 16-byte chunk `ch` of row `row` of the row-major K- tile:
// the chunk index is XORed with the row's low four bits in swapped halves, so
// that the transposed reads hit distinct banks.
__device__ __forceinline__ int sg_off(int row, int ch) {
    return row * 256 + ((ch ^ (((row & 3) << 2) | ((row >> 2) & 3))) << 4);
}
// Fragment-major tile: fragment (rt, kb), this lane's 16 bytes.
__device__ __forceinline__ int fm_off(int rt, int kb) {
    return (4 * rt + kb) * 1024 + (threadIdx.x & 63) * 16;
}

// 8 bf16 as 8 fp32, and back.
__device__ __forceinline__ void unpack8(bf16x8 x, f32x4 &lo, f32x4 &hi) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = (float)x[e];
        hi[e] = (float)x[4 + e];
    }
}
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) { return cat8(cvt4(lo), cvt4(hi)); }

struct SgArgs {
    const __bf16 *k, *v;
    const float *g, *beta, *S0;
    float *S_T;       // segment 0 leaves its final state here
    float *mapN;      // [B*H][nseg-1][K][V]
    float *mapM;      // [B*H][nseg-1][K][K]
    int *mflag;       // [B*H][nseg-1][4]: 0 where chain wave w's M columns are all zero
    int T, H, nseg, seg_len;
};

// Gram block index of (I, J), J <= I: the diagonal blocks first, then
// (1,0) (2,0) (3,0) (2,1) (3,1) (3,2).
__device__ __forceinline__ constexpr int gblk(int I, int J) {
    return I == J ? I : (J == 0 ? 3 + I : (J == 1 ? 5 + I : 9));
}
// -G fragment (and its 8-byte half) that holds block (I, J), J < I, for the
// substitution: F0 = G_10 | 0, F1 = G_20 | G_21, F2 = G_30 | G_31, F3 = G_32 | 0.
__device__ __forceinline__ constexpr int gfrag_off(int I, int J) {
    return I == 1 ? 0 : (I == 2 ? 1024 + 8 * J : (J < 2 ? 2048 + 8 * J : 3072));
}

__global__ __launch_bounds__(SG_NTHR, 1) void chunk_fwd_seg_kernel(SgArgs a)
{
    using L = SgSmem;
    constexpr int K = SG_K;
    constexpr int NKB = K / 32;

    extern __shared__ __attribute__((aligned(256))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r16 = lane & 15;
    const int gq = lane >> 4;

    const int T = a.T, H = a.H;
    // segment-major order: the heads of one segment run at about the same time,
    // so the rows of a token (all heads side by side in memory) are fetched together
    const int nbh = gridDim.x / a.nseg;
    const int seg = blockIdx.x / nbh, bh = blockIdx.x % nbh;
    const int b = bh / H, h = bh % H;
    const long row_base = (long)b * T * H + h;   // row of token 0 in [B*T*H]
    const int nchunks = (T + SG_T - 1) / SG_T;
    const int c0 = seg * a.seg_len, c1 = min(nchunks, c0 + a.seg_len);

    auto hbuf = [&](int c) { return smem + L::oH + (c & 1) * L::HBUF; };
    float *sPart = reinterpret_cast<float *>(smem + L::pPart);
    float *sBeta = reinterpret_cast<float *>(smem + L::pBeta);
    unsigned *ctr = reinterpret_cast<unsigned *>(smem + L::kCtr);
    if (tid == 0) *ctr = 0u;
    lds_barrier();

    if (wave >= 4) {
        // ============================ prep waves ============================
        const int pw = __builtin_amdgcn_readfirstlane(wave - 4);   // key block of this wave
        // This lane: rows 16 rt + r16 of the chunk, keys 32 pw + 8 gq .. +7.
        unsigned loff[4], boff[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            boff[rt] = (unsigned)((16 * rt + r16) * H);
            loff[rt] = boff[rt] * (unsigned)K + (unsigned)(32 * pw + 8 * gq);
        }

        struct Raw {
            bf16x8 k[4];
            f32x4 g[4][2];
            float b[4];
        };
        // Loads of chunk n: always the same number of memory instructions
        // (rows past T read row T-1 and are zeroed: g = beta = k = 0 there,
        // an identity step).
        auto fetch = [&](int n, Raw &r) __attribute__((always_inline)) {
            const int t0 = n * SG_T;
            const int nlive = T - t0;                        // rows of this chunk inside T
            const long rbase = row_base + (long)t0 * H;      // wave-uniform
            const __bf16 *kb = a.k + rbase * K;
            const float *gb = a.g + rbase * K;
            const float *bb = a.beta + rbase;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int row = 16 * rt + r16;
                const bool live = row < nlive;
                const unsigned lo = live ? loff[rt] : (unsigned)((nlive - 1) * H * K + 32 * pw + 8 * gq);
                const unsigned bo = live ? boff[rt] : (unsigned)((nlive - 1) * H);
                r.k[rt] = *reinterpret_cast<const bf16x8 *>(kb + lo);
                r.g[rt][0] = *reinterpret_cast<const f32x4 *>(gb + lo);
                r.g[rt][1] = *reinterpret_cast<const f32x4 *>(gb + lo + 4);
                r.b[rt] = pw == 0 ? bb[bo] : 0.f;   // beta: only wave 0 stages it
            }
        };
        // The loads of token block rt of chunk n only (same addressing as fetch).
        auto fetch_rt = [&](int n, int rt, Raw &r) __attribute__((always_inline)) {
            const int t0 = n * SG_T;
            const int nlive = T - t0;
            const long rbase = row_base + (long)t0 * H;
            const __bf16 *kb = a.k + rbase * K;
            const float *gb = a.g + rbase * K;
            const float *bb = a.beta + rbase;
            const int row = 16 * rt + r16;
            const bool live = row < nlive;
            const unsigned lo = live ? loff[rt] : (unsigned)((nlive - 1) * H * K + 32 * pw + 8 * gq);
            const unsigned bo = live ? boff[rt] : (unsigned)((nlive - 1) * H);
            r.k[rt] = *reinterpret_cast<const bf16x8 *>(kb + lo);
            r.g[rt][0] = *reinterpret_cast<const f32x4 *>(gb + lo);
            r.g[rt][1] = *reinterpret_cast<const f32x4 *>(gb + lo + 4);
            r.b[rt] = pw == 0 ? bb[bo] : 0.f;
        };
        auto zero_dead = [&](int n, Raw &r) __attribute__((always_inline)) {
            const int nlive = T - n * SG_T;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (16 * rt + r16 >= nlive) {
                    r.k[rt] = bf16x8{};
                    r.g[rt][0] = f32x4{0.f, 0.f, 0.f, 0.f};
                    r.g[rt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                    r.b[rt] = 0.f;
                }
            }
        };

        Raw r, nx;
        unsigned arrivals = 0;
        // Chunk n from its raw loads (in nx on entry); issues the v copies of
        // chunk n and, once the tiles are out, the loads of chunk n + 1.
        auto prepare = [&](int n) __attribute__((always_inline)) {
            char *Hb = hbuf(n);
            // The loads of chunk n (issued a period ago) are complete before the
            // v copies go out.  A compiler-visible wait: the compiler's own wait
            // for them would otherwise count the untracked copies too.
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            r = nx;
            zero_dead(n, r);

            // Forward over the four token blocks: lambda (4 DPP scan steps over
            // the block's 16 rows), e^{+-lambda}, the block factor E_rt (row 15),
            // K+ = k e^{lambda} e^{R_rt} to LDS; KL and KI kept as operands.
            f32x4 E[4][2], ki[4][2];
            Frag<__bf16> fKL[4];
            f32x4 ER0 = {1.f, 1.f, 1.f, 1.f}, ER1 = ER0;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 lam[2] = {r.g[rt][0], r.g[rt][1]};
#pragma unroll
                for (int st = 0; st < 4; ++st)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float x = lam[hh][e];
                            lam[hh][e] = x + (st == 0 ? dpp_shr<0x111>(x) : st == 1 ? dpp_shr<0x112>(x)
                                              : st == 2 ? dpp_shr<0x114>(x) : dpp_shr<0x118>(x));
                        }
                f32x4 el[2], ei[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = lam[hh][e] * 1.44269504088896341f;
                        el[hh][e] = __builtin_amdgcn_exp2f(x);
                        ei[hh][e] = __builtin_amdgcn_exp2f(-x);
                        E[rt][hh][e] = lane_in_row<15>(el[hh][e]);
                    }
                f32x4 k0, k1;
                unpack8(r.k[rt], k0, k1);
                // this block's raw registers are consumed: the same block of the
                // next chunk goes in flight (four loads per block, spread over the
                // loop rather than issued as one burst)
                GDN_SCHED_FENCE();
                if (n + 1 < c1) fetch_rt(n + 1, rt, nx);
                GDN_SCHED_FENCE();
                const f32x4 kl0 = k0 * el[0], kl1 = k1 * el[1];
                ki[rt][0] = k0 * ei[0];
                ki[rt][1] = k1 * ei[1];
                fKL[rt].v = pack8(kl0, kl1);
                *reinterpret_cast<bf16x8 *>(Hb + L::hKP + fm_off(rt, pw)) = pack8(kl0 * ER0, kl1 * ER1);
                ER0 *= E[rt][0];
                ER1 *= E[rt][1];
            }
            // Backward: K- = KI e^{gn - R_rt} = KI E_rt ... E_3; e^{gn} at the end.
            {
                f32x4 ES0 = {1.f, 1.f, 1.f, 1.f}, ES1 = ES0;
#pragma unroll
                for (int rt = 3; rt >= 0; --rt) {
                    ES0 *= E[rt][0];
                    ES1 *= E[rt][1];
                    *reinterpret_cast<bf16x8 *>(Hb + L::hKM + sg_off(16 * rt + r16, 4 * pw + gq)) =
                        pack8(ki[rt][0] * ES0, ki[rt][1] * ES1);
                }
                if (r16 == 0) {
                    float *go = reinterpret_cast<float *>(Hb + L::hEgn) + 32 * pw + 8 * gq;
                    *reinterpret_cast<f32x4 *>(go) = ES0;
                    *reinterpret_cast<f32x4 *>(go + 4) = ES1;
                }
            }
            if (pw == 0 && gq == 0) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) sBeta[16 * rt + r16] = r.b[rt];
            }
            // This key block's share of the ten Gram blocks, G_IJ over keys
            // 32 pw .. +31, computed transposed (rows s of block J, columns t of
            // block I): A = KI_J F_IJ (F_IJ = E_J .. E_{I-1} per key), B = KL_I.
            {
                float *mine = sPart + pw * 10 * 256 + lane * 4;
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    f32x4 f0 = {1.f, 1.f, 1.f, 1.f}, f1 = f0;
#pragma unroll
                    for (int I = J; I < 4; ++I) {
                        if (I > J) {
                            f0 *= E[I - 1][0];
                            f1 *= E[I - 1][1];
                        }
                        const Frag<__bf16> fa = {pack8(ki[J][0] * f0, ki[J][1] * f1)};
                        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                        const f32x4 part = mma(z, fa, fKL[I]);
                        *reinterpret_cast<f32x4 *>(mine + gblk(I, J) * 256) = part;
                    }
                }
            }
            arrivals += 4;
            prep_barrier(ctr, arrivals);   // every share and beta written

            // Sum the four shares of this wave's blocks: the diagonal block pw
            // (then T'_pw), and -G of p0: (1,0) (3,0)   p1: (2,1) (3,1)
            // p2: (3,2)   p3: (2,0).
            auto sum4 = [&](int blk) __attribute__((always_inline)) {
                f32x4 s4[4];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    s4[w] = *reinterpret_cast<const f32x4 *>(sPart + (w * 10 + blk) * 256 + lane * 4);
                return (s4[0] + s4[1]) + (s4[2] + s4[3]);
            };
            auto offdiag = [&](auto ic, auto jc) __attribute__((always_inline)) {
                constexpr int I = decltype(ic)::value, J = decltype(jc)::value;
                const f32x4 gsum = sum4(gblk(I, J));
                *reinterpret_cast<bf16x4 *>(Hb + L::hAn + gfrag_off(I, J) + lane * 16) = cvt4(-gsum);
            };
            {
                // lane (gq, j = r16) holds G[t = 16 pw + j][s = 16 pw + 4 gq + e]:
                // -A[t][s] = -beta_t G[t][s] (s < t) goes to this wave's scratch
                // row-major, the row-wise inverse reads it back in order
                const f32x4 gsum = sum4(gblk(pw, pw));
                const float bt = sBeta[16 * pw + r16];
                float *sAd = reinterpret_cast<float *>(smem + L::pAd) + pw * 256;
                f32x4 na;
#pragma unroll
                for (int e = 0; e < 4; ++e) na[e] = (4 * gq + e < r16) ? -bt * gsum[e] : 0.f;
                *reinterpret_cast<f32x4 *>(sAd + r16 * 16 + 4 * gq) = na;
                const f32x4 tr = unit_lower_inverse16_rows(sAd);   // lane 4j + p: T[j][4p .. 4p+3]
                const f32x4 bs = *reinterpret_cast<const f32x4 *>(sBeta + 16 * pw + 4 * (lane & 3));
                *reinterpret_cast<bf16x4 *>(Hb + L::hTd + ((16 * pw + (lane >> 2)) * L::LDD + 4 * (lane & 3)) * 2) =
                    cvt4(tr * bs);
            }
            using std::integral_constant;
            if (pw == 0) {
                offdiag(integral_constant<int, 1>(), integral_constant<int, 0>());
                offdiag(integral_constant<int, 3>(), integral_constant<int, 0>());
            } else if (pw == 1) {
                offdiag(integral_constant<int, 2>(), integral_constant<int, 1>());
                offdiag(integral_constant<int, 3>(), integral_constant<int, 1>());
            } else if (pw == 2) {
                offdiag(integral_constant<int, 3>(), integral_constant<int, 2>());
            } else {
                offdiag(integral_constant<int, 2>(), integral_constant<int, 0>());
            }
        };

        if (c0 < c1) {
            fetch(c0, nx);
            prepare(c0);
            lds_barrier();                      // chunk c0 is ready
        }
        for (int c = c0; c < c1; ++c) {
            if (c + 1 < c1) prepare(c + 1);
            lds_barrier();
        }
        wait_vm<0>();   // nothing in flight at exit
        return;
    }

    // ============================= chain waves =============================
    // Column groups (16 columns each) of this wave: groups 0 and 1 hold columns
    // 32 wave + 16 cg + r16 of N (of the state itself in segment 0), groups 2 and
    // 3 the same columns of M (later segments only).  Accumulator S[cg][ct],
    // ct = 2 kb + hh, element e holds the row of key 32 kb + 8 gq + 4 hh + e.
    const int cw = wave;
    auto key_of = [&](int ct, int e) { return 32 * (ct >> 1) + 8 * gq + 4 * (ct & 1) + e; };
    auto col_of = [&](int cg) { return 32 * cw + 16 * (cg & 1) + r16; };
    // M' = Diag(e^{gn}) M - K-^T D(K+ M) is exactly zero once M is (every product
    // and sum is of zeros), so a wave skips its M columns from the chunk after
    // they are all seen to be zero; the decay gets them there within a few
    // chunks unless the gates stay close to 1.
    bool mlive = seg > 0;
    f32x4 S[4][8];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
        const int col = col_of(cg);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x = 0.f;
                if (cg < 2) {
                    if (seg == 0 && a.S0) x = a.S0[((long)bh * K + key_of(ct, e)) * K + col];
                } else if (seg > 0) {
                    x = key_of(ct, e) == col ? 1.f : 0.f;
                }
                S[cg][ct][e] = x;
            }
    }

    // per-lane LDS offsets that do not change between chunks
    const int trow = 4 * gq + (r16 >> 2), tq = r16 & 3;
    int k_tr[NKB];
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) k_tr[kk] = sg_off(trow, 4 * kk + tq);
    // v in the accumulator layout from the fragment-major tile: lane 4i + a of a
    // 16-lane group addresses token 4 gq + i, columns 16 cgv + 4 a .. +3
    int v_tr[4];
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
        const int cgv = 2 * cw + (cg & 1);   // groups 2 and 3 (M) read no v
        v_tr[cg] = (cgv >> 1) * 1024 + (16 * (2 * (cgv & 1) + (tq >> 1)) + trow) * 16 + 8 * (tq & 1);
    }

    // v copies: this wave fills the four fragments of token block cw of a
    // chunk, lane (gq, r16) the 16 bytes of token 16 cw + r16, columns
    // 32 cb + 8 gq .. +7; a chunk's copies go out a period ahead and land
    // before the hand-over barrier
    unsigned voff[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) voff[cb] = 2u * (unsigned)((16 * cw + r16) * H * K + 32 * cb + 8 * gq);
    auto copy_v = [&](int n) __attribute__((always_inline)) {
        char *dst = hbuf(n) + L::hV + 4 * cw * 1024;
        const int t0 = n * SG_T;
        if (t0 + SG_T <= T) {
            const __bf16 *vb = a.v + (row_base + (long)t0 * H) * K;   // wave-uniform
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) g2lds16s(vb, voff[cb], dst + cb * 1024);
        } else {
            const int t = min(t0 + 16 * cw + r16, T - 1);
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                g2lds16(a.v + (row_base + (long)t * H) * K + 32 * cb + 8 * gq, dst + cb * 1024);
        }
    };
    if (c0 < c1) {
        copy_v(c0);
        wait_vm<0>();
        lds_barrier();                      // chunk c0 is ready
    }

    for (int c = c0; c < c1; ++c) {
        if (c + 1 < c1) copy_v(c + 1);
        {
            const char *Hb = hbuf(c);
            const char *sKP = Hb + L::hKP;
            const unsigned vbase = lds_u32(Hb + L::hV);
            const char *sAn = Hb + L::hAn;
            const __bf16 *sTd = reinterpret_cast<const __bf16 *>(Hb + L::hTd);
            const float *sEgn = reinterpret_cast<const float *>(Hb + L::hEgn);
            unsigned ktr_addr[NKB];
#pragma unroll
            for (int kk = 0; kk < NKB; ++kk) ktr_addr[kk] = opaque(lds_u32(Hb + L::hKM) + k_tr[kk]);

            // Phases A and B, one 16-column tile at a time: X = V - K+ S (V = 0
            // in the columns of M), then the block forward substitution
            // D_i = T'_ii (X_i - sum_{j<i} G_ij D_j) (-G stored).
            Frag<__bf16> Df[4][2];
#pragma unroll
            for (int cg = 0; cg < 4; ++cg) {
                if (cg >= 2 && !mlive) continue;
                Frag<__bf16> Sf[NKB];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) Sf[kb] = reg_frag<__bf16>(S[cg][2 * kb], S[cg][2 * kb + 1]);
                f32x4 X[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    Frag<__bf16> fk[NKB];
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) fk[kb] = {*reinterpret_cast<const bf16x8 *>(sKP + fm_off(rt, kb))};
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) acc = mma(acc, fk[kb], Sf[kb]);
                    X[rt] = acc;
                }
                GDN_SCHED_FENCE();
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if (cg < 2) {
                        const bf16x4 vv = lds_read_tr(vbase + v_tr[cg] + 4096 * rt);
#pragma unroll
                        for (int e = 0; e < 4; ++e) X[rt][e] = (float)vv[e] - X[rt][e];
                    } else {
                        X[rt] = -X[rt];
                    }
                }
                const bf16x4 zz = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
                auto lo_frag = [&](int off) __attribute__((always_inline)) {
                    return Frag<__bf16>{cat8(*reinterpret_cast<const bf16x4 *>(sAn + off + lane * 16), zz)};
                };
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                f32x4 Dd[4];
                Dd[0] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 0, 0), reg_frag<__bf16>(X[0], z));
                f32x4 Y = mma_lo(X[1], lo_frag(0), reg_frag<__bf16>(Dd[0], z));
                Dd[1] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 16, 0), reg_frag<__bf16>(Y, z));
                Df[cg][0] = reg_frag<__bf16>(Dd[0], Dd[1]);
                Y = mma(X[2], Frag<__bf16>{*reinterpret_cast<const bf16x8 *>(sAn + 1024 + lane * 16)}, Df[cg][0]);
                f32x4 Y3 = mma(X[3], Frag<__bf16>{*reinterpret_cast<const bf16x8 *>(sAn + 2048 + lane * 16)}, Df[cg][0]);
                Dd[2] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 32, 0), reg_frag<__bf16>(Y, z));
                Y3 = mma_lo(Y3, lo_frag(3072), reg_frag<__bf16>(Dd[2], z));
                Dd[3] = mma_lo(z, lds_frag_lo(sTd, L::LDD, 48, 0), reg_frag<__bf16>(Y3, z));
                Df[cg][1] = reg_frag<__bf16>(Dd[2], Dd[3]);
            }

            // Phase D: S' = Diag(e^{gn}) S + K-^T D for all 64 columns, the k^T
            // fragments of each key tile read once.
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const unsigned pk = ktr_addr[ct >> 1] + 8 * (ct & 1);
                bf16x4 kt[4];
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) {
                    kt[2 * kb2] = lds_read_tr(pk + 256 * 32 * kb2);
                    kt[2 * kb2 + 1] = lds_read_tr(pk + 256 * (32 * kb2 + 16));
                }
                const f32x4 eg = *reinterpret_cast<const f32x4 *>(sEgn + key_of(ct, 0));
#pragma unroll
                for (int cg = 0; cg < 4; ++cg) {
                    if (cg >= 2 && !mlive) continue;
                    f32x4 s = S[cg][ct] * eg;
#pragma unroll
                    for (int kb2 = 0; kb2 < 2; ++kb2)
                        s = mma(s, Frag<__bf16>{cat8(kt[2 * kb2], kt[2 * kb2 + 1])}, Df[cg][kb2]);
                    S[cg][ct] = s;
                }
            }
            if (mlive && (c & 3) == 3) {     // every fourth chunk: are the M columns all zero?
                unsigned bits = 0u;
#pragma unroll
                for (int cg = 2; cg < 4; ++cg)
#pragma unroll
                    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e) bits |= __float_as_uint(S[cg][ct][e]) & 0x7fffffffu;
                mlive = __builtin_amdgcn_ballot_w64(bits != 0u) != 0ull;
            }
        }
        wait_vm<0>();                        // the next chunk's v landed
        lds_barrier();
    }

    float *dN, *dM = nullptr;
    if (seg == 0) {
        dN = a.S_T + (long)bh * K * K;
    } else {
        const long slot = (long)bh * (a.nseg - 1) + (seg - 1);
        dN = a.mapN + slot * K * K;
        dM = a.mapM + slot * K * K;
        // M columns seen to be all zero are not written; the combine skips them
        if (lane == 0) a.mflag[slot * 4 + cw] = mlive ? 1 : 0;
    }
#pragma unroll
    for (int cg = 0; cg < 4; ++cg) {
        if (cg >= 2 && (seg == 0 || !mlive)) continue;
        float *dst = cg < 2 ? dN : dM;
        const int col = col_of(cg);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[key_of(ct, e) * K + col] = S[cg][ct][e];
    }
}

// ---------------------------------------------------------------------------
// Combine: for each head, S <- M_s S + N_s over segments s = 1 .. nseg-1 in
// order, starting from segment 0's final state in S_T; fp32 matrix cores
// (16 x 16 x 4).  One workgroup of 4 waves per (head, 16 value columns): wave
// w computes rows 32 w .. 32 w + 31; the state block lives in LDS between steps.
// With Sb, the state entering each segment s >= 1 is also written there
// ([B*H][nseg-1][K][V]): the incoming states of the o pass.
struct SgCombArgs {
    const float *mapN, *mapM;
    const int *mflag;   // [nbh][nseg-1][4]: 0 where columns 32 w .. 32 w + 31 of M_s are all zero (not written)
    float *S_T;
    float *Sb;
    int nseg, xcd_map;
    long nbh;
};

__global__ __launch_bounds__(256) void seg_combine_kernel(SgCombArgs a)
{
    constexpr int K = SG_K, V = SG_K, NCB = V / 16, LDS_LD = 16 + 4;
    __shared__ float sS[K * LDS_LD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, gq = lane >> 4;
    long bh;
    int cb;
    {
        const long w = blockIdx.x;
        if (a.xcd_map) {   // the column blocks of one head on one XCD (shared M_s in its L2)
            const long xcd = w & 7, slot = w >> 3;
            cb = (int)(slot % NCB);
            bh = (slot / NCB) * 8 + xcd;
        } else {
            bh = w / NCB;
            cb = (int)(w % NCB);
        }
    }
    float *ST = a.S_T + bh * K * V;
    for (int i = tid; i < K * 16; i += 256) sS[(i >> 4) * LDS_LD + (i & 15)] = ST[(i >> 4) * V + 16 * cb + (i & 15)];
    __syncthreads();
    const int col = 16 * cb + r16;
    for (int s = 1; s < a.nseg; ++s) {
        const long slot = bh * (a.nseg - 1) + (s - 1);
        const float *Mp = a.mapM + slot * K * K;
        const float *Np = a.mapN + slot * K * V;
        if (a.Sb) {
            float *Bp = a.Sb + slot * K * V;
            for (int i = tid; i < K * 16; i += 256) Bp[(i >> 4) * V + 16 * cb + (i & 15)] = sS[(i >> 4) * LDS_LD + (i & 15)];
        }
        f32x4 acc[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rt][e] = Np[(32 * wave + 16 * rt + 4 * gq + e) * V + col];
        // columns 16 m .. 16 m + 15 of M_s: skipped where the segment kernel found
        // them all zero (they contribute nothing and were not written)
        int live[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) live[w] = __builtin_amdgcn_readfirstlane(a.mflag[slot * 4 + w]);
        f32x4 am[8][2];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (!live[m >> 1]) continue;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                am[m][rt] = *reinterpret_cast<const f32x4 *>(Mp + (32 * wave + 16 * rt + r16) * K + 16 * m + 4 * gq);
        }
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            if (!live[m >> 1]) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float bv = sS[(16 * m + 4 * gq + e) * LDS_LD + r16];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) acc[rt] = mfma_f32(am[m][rt][e], bv, acc[rt]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sS[(32 * wave + 16 * rt + 4 * gq + e) * LDS_LD + r16] = acc[rt][e];
        __syncthreads();
    }
    for (int i = tid; i < K * 16; i += 256) ST[(i >> 4) * V + 16 * cb + (i & 15)] = sS[(i >> 4) * LDS_LD + (i & 15)];
}

// ---------------------------------------------------------------------------
// Host side.

// Segments per (b, h) for the sequence-parallel form, or 1 when the call should
// run the sequential kernel: long sequences with too few heads to fill the
// chip.  Enough segments for about three workgroups per CU of a 256-CU part,
// at least 8 chunks per segment (shorter ones would spend more on the maps and
// their combine than they save), at most 64 segments (the combine walks them
// in order).
int chunk_fwd_seg_count(long B, long T, long H)
{
    const long nch = (T + SG_T - 1) / SG_T;
    const long bh = B * H;
    if (bh <= 0 || nch <= 0 || bh * 2 >= 256) return 1;
    long nseg = (768 + bh - 1) / bh;
    nseg = nseg < nch / 8 ? nseg : nch / 8;
    nseg = nseg < 64 ? nseg : 64;
    if (nseg < 2) return 1;
    // equal whole-chunk segments, none empty
    const long len = (nch + nseg - 1) / nseg;
    return (int)((nch + len - 1) / len);
}

// The segment maps (N and M per later segment) and, for a call that also
// writes o, the incoming state of every later segment.
unsigned long long chunk_fwd_seg_workspace(long B, long H, int nseg, bool want_o)
{
    if (nseg <= 1) return 0;
    // N and M (and the incoming states) in fp32, then four int flags per map
    return (unsigned long long)B * H * (nseg - 1) * ((want_o ? 3ull : 2ull) * SG_K * SG_K + 4ull) * 4ull;
}

hipError_t chunk_fwd_wsc_seg_launch(const void *q, const void *k, const void *v, const float *g,
                                    const float *beta, const float *S0, const float *Sb, void *o,
                                    int B, int T, int H, int nseg, int seg_len, hipStream_t st);

// Device scratch of the entry point that allocates nothing: the segment maps of
// one call live here instead of in a caller's workspace.  Host code never
// passes this name to a kernel: it is a host-side stand-in, so its device
// address is looked up once per device (seg_scratch) and that pointer is used.
constexpr unsigned long long SG_SCRATCH_BYTES = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[SG_SCRATCH_BYTES];

unsigned long long chunk_fwd_seg_scratch_bytes() { return SG_SCRATCH_BYTES; }

// The device address of `scratch` on the current device, looked up on the
// first call for each device (with that device current) and kept.
hipError_t seg_scratch(void **p)
{
    constexpr int MAXDEV = 64;
    static std::mutex mu;
    static void *addr[MAXDEV] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = ptr;
    }
    *p = addr[dev];
    return hipSuccess;
}

// q and o: null for a final-state-only call; with o, a third launch runs every
// segment's outputs from the incoming states the combine wrote.
hipError_t chunk_fwd_seg_launch(const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *S0, void *o, float *S_T, void *ws,
                                int B, int T, int H, int nseg, hipStream_t st)
{
    using L = SgSmem;
    static bool attr_set = false;  // benign race: every thread sets the same value
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)chunk_fwd_seg_kernel,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const long nch = (T + SG_T - 1) / SG_T;
    const long bh = (long)B * H;
    SgArgs a;
    a.k = (const __bf16 *)k; a.v = (const __bf16 *)v; a.g = g; a.beta = beta; a.S0 = S0;
    a.S_T = S_T;
    a.seg_len = (int)((nch + nseg - 1) / nseg);
    a.nseg = nseg;
    a.mapN = (float *)ws;
    a.mapM = a.mapN + bh * (nseg - 1) * SG_K * SG_K;
    a.mflag = (int *)(a.mapM + bh * (nseg - 1) * SG_K * SG_K * (o ? 2 : 1));   // after M (and Sb)
    a.T = T; a.H = H;
    hipLaunchKernelGGL(chunk_fwd_seg_kernel, dim3((unsigned)(bh * nseg)), dim3(SG_NTHR), L::bytes, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nseg == 1) return e;
    SgCombArgs c;
    c.mapN = a.mapN; c.mapM = a.mapM; c.mflag = a.mflag; c.S_T = S_T; c.nseg = nseg; c.nbh = bh;
    c.Sb = o ? a.mapM + bh * (nseg - 1) * SG_K * SG_K : nullptr;
    c.xcd_map = bh % 8 == 0 ? 1 : 0;
    hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(bh * (SG_K / 16))), dim3(256), 0, st, c);
    e = hipGetLastError();
    if (e != hipSuccess || !o) return e;
    return chunk_fwd_wsc_seg_launch(q, k, v, g, beta, S0, c.Sb, o, B, T, H, nseg, a.seg_len, st);
}

} // namespace gdn
