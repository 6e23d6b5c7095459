// prologue.h -- arguments of the prologue kernels (prologue.hip), shared with the
// C ABI (gdn_api.cpp).
#pragma once
#include <hip/hip_runtime.h>

namespace gdn {

// gdn_prologue: raw [B,T,H,*] in, prologue-applied [B,T,H,*] out.  Carried
// convolution states [B,3,H*K] / [B,3,H*V] in the input dtype (null: zeros in,
// not written out).
struct PrArgs {
    const void *q_raw, *k_raw, *v_raw;
    const float *g_raw, *b_raw;
    const float *w_q, *w_k, *w_v;          // [H*K,4], [H*K,4], [H*V,4]
    const void *cs_q, *cs_k, *cs_v;
    void *q, *k, *v;
    float *g, *beta;
    void *cs_q_out, *cs_k_out, *cs_v_out;
    float cap;
    int B, T, H;
};

// gdn_recurrent_step_prologue: one token of N sequences from the raw projections.
struct RpArgs {
    const void *q_raw, *k_raw, *v_raw;     // [N,H,K] / [N,H,V]
    const float *g_raw, *b_raw;            // [N,H(,K)] / [N,H]
    const float *w_q, *w_k, *w_v;
    const void *cs_q, *cs_k, *cs_v;        // [N,3,H*K] / [N,3,H*V] or null
    void *cs_q_out, *cs_k_out, *cs_v_out;  // or null; never the inputs
    float *S;                              // [N,H,K,V], in place
    void *o;                               // [N,H,V] or null
    float cap;
    int H;
};

hipError_t prologue_launch(bool bf16, bool channel, bool silu, int K, int V, const PrArgs &a,
                           hipStream_t st);
hipError_t step_prologue_launch(bool bf16, bool channel, bool silu, int K, int V, const RpArgs &a,
                                long nslices, hipStream_t st);

} // namespace gdn
