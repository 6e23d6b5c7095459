// chunk_bwd.h -- arguments and workspace layout of the chunkwise backward
// (chunk_bwd.hip), shared with the C ABI (gdn_api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// value columns per workgroup in the two state sweeps
constexpr int BW_VB = 32;

// Intermediates, each an array over the B*H*ceil(T/64) chunks (chunk
// ci = (b H + h) NC + c).  fp32, rows of a chunk contiguous, except where
// marked F: fragment order (the matrix-core operand layout of the sweeps); A:
// accumulator-tile order (the layout of a matrix-core result); and S: the
// sweeps' operands, fragment order in the input dtype (bf16 inputs use half of
// the fp32-sized slot; the last three arrays are used by bf16 only):
struct BwWs {
    float *gam;   // [64][K]  in-chunk cumulative log-decay
    float *Tm;    // [64][64] (I + diag(beta) G)^{-1}                          F
    float *TT;    // [64][64] its transpose                                     F
    float *Gm;    // [64][64] G, strictly lower (bf16 for bf16 inputs)
    float *PT;    // [64][64] P^T (P lower with the diagonal)                     S
    float *hS;    // [K][V]   state entering the chunk                      (input dtype)
    float *dhS;   // [K][V]   dL/d(state leaving the chunk)                 (input dtype)
    float *Dl;    // [64][V]  Delta
    float *dDl;   // [64][V]  dL/dDelta
    float *dQp;   // [64][K]  dL/dQp (then d gamma)                           A
    float *dKm;   // [64][K]  dL/dKm                                            A
    float *dWn;   // [64][K]  dDelta S^T (then Z = -T^T of it)                A
    float *dP;    // [64][64] dO Delta^T                                        A
    float *dT;    // [64][64] dDelta (beta V)^T (then dG)                       A
    float *dgn;   // [K]      e^{gn} rowsum(S * dS')
    float *Kp;    // [64][K]  k e^{gamma}                                       F
    float *Km;    // [64][K]  k e^{gn - gamma}                                  S
    float *KpT;   // [K][64]  Kp^T                                              S
    float *KmT;   // [K][64]  Km^T                                              S
    float *QpT;   // [K][64]  (q e^{gamma})^T                                   S
    float *egn;   // [K]      e^{gn}
    float *Kps;   // [64][K]  Kp                                                S, bf16
    float *Tms;   // [64][64] T                                                 S, bf16
    float *TTs;   // [64][64] T^T                                               S, bf16
};

struct BwArgs {
    const void *q, *k, *v, *d_o;             // [B,T,H,K] / [B,T,H,V], input dtype
    const float *g, *beta, *S0, *dS_T;       // S0, dS_T may be null (zeros)
    void *dq, *dk, *dv;                      // input dtype
    float *dg, *dbeta, *dS0;                 // dS0 may be null (not wanted)
    BwWs ws;
    int T, H, NC;
    int NS;                                  // slices, B * H
};

// Byte size of the workspace for nchunks chunks; with base != null also fills
// ws with the array addresses (each array 256-byte aligned from base).
inline unsigned long long bw_workspace(unsigned long long nchunks, int K, int V, void *base,
                                       BwWs *ws)
{
    const unsigned long long C = 64, Ku = (unsigned)K, Vu = (unsigned)V;
    constexpr int NA = 24;
    const unsigned long long per[NA] = {C * Ku, C * C, C * C, C * C, C * C, Ku * Vu, Ku * Vu,
                                        C * Vu, C * Vu, C * Ku, C * Ku, C * Ku, C * C, C * C,
                                        Ku, C * Ku, C * Ku, C * Ku, C * Ku, C * Ku, Ku,
                                        C * Ku / 2, C * C / 2, C * C / 2};
    float **dst[NA] = {nullptr};
    if (ws) {
        float **p[NA] = {&ws->gam, &ws->Tm, &ws->TT, &ws->Gm, &ws->PT, &ws->hS, &ws->dhS,
                         &ws->Dl, &ws->dDl, &ws->dQp, &ws->dKm, &ws->dWn, &ws->dP, &ws->dT,
                         &ws->dgn, &ws->Kp, &ws->Km, &ws->KpT, &ws->KmT, &ws->QpT,
                         &ws->egn, &ws->Kps, &ws->Tms, &ws->TTs};
        for (int i = 0; i < NA; ++i) dst[i] = p[i];
    }
    unsigned long long off = 0;
    for (int i = 0; i < NA; ++i) {
        if (ws && base) *dst[i] = reinterpret_cast<float *>(static_cast<char *>(base) + off);
        off += (nchunks * per[i] * 4 + 255) / 256 * 256;
    }
    return off;
}

hipError_t chunk_bwd_launch(bool bf16, bool channel, int K, int V, const BwArgs &a, long nslices,
                            hipStream_t st);

} // namespace gdn
