// prologue_ops.h -- per-element steps of the prologue (between the projections
// and the recurrence), shared by the standalone prologue kernels and the chunk
// kernel that runs them in its load stage.
//   activation  SiLU after the kernel-4 convolution (optional)
//   q, k        divided by their L2 norm over the head's K channels
//   g           -min(softplus(g_raw), cap)   (cap 5: Atomic-GDN2 card, section 2.1)
//   beta        sigmoid(b_raw)
#pragma once
#include "gdn_common.h"

namespace gdn {

// The hardware reciprocal and reciprocal square root (1 ulp) rather than
// IEEE-exact division: with exact division the chunk-mode prologue was bound by
// its VALU work (about ten instructions per division, nine divisions per token
// and thread), not by HBM.
__device__ __forceinline__ float pr_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float pr_sigmoid(float x) { return pr_rcp(1.f + __expf(-x)); }
__device__ __forceinline__ float pr_silu(float x) { return x * pr_rcp(1.f + __expf(-x)); }
// 1 / max(sqrt(ss), 1e-12) for ss >= 0
__device__ __forceinline__ float pr_rnorm(float ss) { return __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f)); }
// -min(softplus(x), cap), softplus evaluated as max(x, 0) + log(1 + e^{-|x|})
__device__ __forceinline__ float pr_gate(float x, float cap)
{
    const float sp = fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x)));
    return -fminf(sp, cap);
}
// One output of the causal 4-tap convolution: taps w[0..3] on tokens
// t-3 .. t (x3 = token t), accumulated in that order.
__device__ __forceinline__ float pr_conv4(const f32x4 &w, float x0, float x1, float x2, float x3)
{
    float v = w[0] * x0;
    v = fmaf(w[1], x1, v);
    v = fmaf(w[2], x2, v);
    return fmaf(w[3], x3, v);
}

} // namespace gdn
