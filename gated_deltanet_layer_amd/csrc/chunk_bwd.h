// chunk_bwd.h -- arguments and workspace layout of the chunkwise backward
// (chunk_bwd.hip), shared with the C ABI (gdn_api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// value columns per workgroup in the two state sweeps (K x VB = 2048 floats)
constexpr int bw_vb(int K) { return 2048 / K; }

// fp32 intermediates, each an array over the B*H*ceil(T/64) chunks
// (chunk ci = (b H + h) NC + c), rows of a chunk contiguous:
struct BwWs {
    float *gam;   // [64][K]  in-chunk cumulative log-decay
    float *Tm;    // [64][64] (I + diag(beta) G)^{-1}
    float *Gm;    // [64][64] G, strictly lower
    float *Pm;    // [64][64] P, lower with the diagonal
    float *hS;    // [K][V]   state entering the chunk
    float *dhS;   // [K][V]   dL/d(state leaving the chunk)
    float *Dl;    // [64][V]  Delta
    float *dDl;   // [64][V]  dL/dDelta
    float *dQp;   // [64][K]  dL/dQp (then d gamma)
    float *dKm;   // [64][K]  dL/dKm
    float *dWn;   // [64][K]  dDelta S^T (then Z = -T^T of it)
    float *dP;    // [64][64] dO Delta^T
    float *dT;    // [64][64] dDelta (beta V)^T
    float *dgn;   // [K]      e^{gn} rowsum(S * dS')
    float *dbv;   // [64]     rowsum(V * T^T dDelta)
};

struct BwArgs {
    const void *q, *k, *v, *d_o;             // [B,T,H,K] / [B,T,H,V], input dtype
    const float *g, *beta, *S0, *dS_T;       // S0, dS_T may be null (zeros)
    void *dq, *dk, *dv;                      // input dtype
    float *dg, *dbeta, *dS0;                 // dS0 may be null (not wanted)
    BwWs ws;
    int T, H, NC;
};

// Byte size of the workspace for nchunks chunks; with base != null also fills
// ws with the array addresses (each array 256-byte aligned from base).
inline unsigned long long bw_workspace(unsigned long long nchunks, int K, int V, void *base,
                                       BwWs *ws)
{
    const unsigned long long C = 64, Ku = (unsigned)K, Vu = (unsigned)V;
    const unsigned long long per[15] = {C * Ku, C * C, C * C, C * C, Ku * Vu, Ku * Vu, C * Vu,
                                        C * Vu, C * Ku, C * Ku, C * Ku, C * C, C * C, Ku, C};
    float **dst[15] = {nullptr};
    if (ws) {
        float **p[15] = {&ws->gam, &ws->Tm, &ws->Gm, &ws->Pm, &ws->hS, &ws->dhS, &ws->Dl,
                         &ws->dDl, &ws->dQp, &ws->dKm, &ws->dWn, &ws->dP, &ws->dT, &ws->dgn,
                         &ws->dbv};
        for (int i = 0; i < 15; ++i) dst[i] = p[i];
    }
    unsigned long long off = 0;
    for (int i = 0; i < 15; ++i) {
        if (ws && base) *dst[i] = reinterpret_cast<float *>(static_cast<char *>(base) + off);
        off += (nchunks * per[i] * 4 + 255) / 256 * 256;
    }
    return off;
}

hipError_t chunk_bwd_launch(bool bf16, bool channel, int K, int V, const BwArgs &a, long nslices,
                            hipStream_t st);

} // namespace gdn
