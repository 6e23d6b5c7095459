// ws_common.h -- device helpers of the warp-specialised chunkwise kernels
// (gfx950): LDS layouts and reads, direct global-to-LDS copies, the prep-wave
// barrier, the row-wise 16 x 16 unit-triangular inverse and Gram products.
#pragma once
#include "mfma_frag.h"
#include <stdint.h>

namespace gdn {

// Scheduling fence: the compiler moves no instruction across it.
#define GDN_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Byte offset of the 16-byte chunk `ch` of q/k row `row` (rows of CPR chunks,
// chunk index XOR-swizzled by the row).
template <int CPR> __device__ __forceinline__ int qk_off(int row, int ch) {
    return row * CPR * 16 + ((ch ^ (row & (CPR - 1))) << 4);
}
// Byte offset of the 16-byte chunk `ch` of v row `row` (8 chunks per row).
__device__ __forceinline__ int v_off(int row, int ch) { return row * 128 + ((ch ^ (row & 7)) << 4); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
// gfx950 transposing LDS read: inside each 16-lane group, lane 4a+b receives
// element b of the 8-byte pieces addressed by lanes a, 4+a, 8+a and 12+a.
// `addr` is an LDS byte address; a constant added to it folds into the
// instruction's offset field.
__device__ __forceinline__ bf16x4 lds_read_tr(unsigned addr) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(uintptr_t)addr);
    return __builtin_bit_cast(bf16x4, r);
}
// 32-bit LDS address of a pointer into shared memory.
__device__ __forceinline__ unsigned lds_u32(const char *p) {
    return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
}
// Keeps the compiler from merging constant offsets into x (so that they stay
// foldable into the LDS instructions that use x).
__device__ __forceinline__ unsigned opaque(unsigned x) {
    asm("" : "+v"(x));
    return x;
}

// q/k fragment: rows row0 + r16, keys 32 kb + 8 gq .. +7 (one 16-byte read).
template <int CPR> __device__ __forceinline__ Frag<__bf16> qk_frag(const char *M, int row0, int kb) {
    return {*reinterpret_cast<const bf16x8 *>(M + qk_off<CPR>(row0 + lane_r16(), 4 * kb + lane_gq()))};
}

// Copies from global memory straight into LDS (global_load_lds): lane l of
// the wave writes its 16 (or 4) bytes from `src` (per lane) at lds + 16 l (or
// + 4 l); `lds` is wave-uniform and goes through M0.  Written as inline asm so
// that the compiler's own wait-count tracking, which would otherwise wait for
// every copy in flight before any LDS access, leaves them alone: the kernel
// waits for them explicitly (wait_vm) before their data is read.  They have no
// register results.
__device__ __forceinline__ unsigned lds_addr(const char *lds) {
    return (unsigned)__builtin_amdgcn_readfirstlane(
        (int)(uintptr_t)(__attribute__((address_space(3))) const char *)lds);
}
__device__ __forceinline__ void g2lds16(const void *src, char *lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 ::"v"(src), "s"(lds_addr(lds)) : "memory", "m0");
}
// Same, from a wave-uniform base (held in SGPRs) plus a 32-bit per-lane byte
// offset: no 64-bit address per lane.
// `base` must be the same in every lane (it is read from the first active one).
__device__ __forceinline__ void g2lds16s(const void *base, unsigned off, char *lds) {
    const unsigned long long b = (unsigned long long)(uintptr_t)base;
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
    const void *sb = (const void *)(uintptr_t)(((unsigned long long)hi << 32) | lo);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(off), "s"(sb), "s"(lds_addr(lds)) : "memory", "m0");
}
__device__ __forceinline__ void g2lds4(const void *src, char *lds) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 ::"v"(src), "s"(lds_addr(lds)) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order).
template <int N> __device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Barrier among the prep waves of a workgroup: each wave adds one arrival to an
// LDS counter and waits until the counter reaches `target` (the number of prep
// waves per use).  Every prep wave reaches every use unconditionally.  The wait is bounded: after ~2^22
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

// Wait (bounded, like prep_barrier) until the arrival counter reaches
// `target`, without arriving.
__device__ __forceinline__ void wait_arrivals(unsigned *ctr, unsigned target) {
    for (int it = 0; it < (1 << 22); ++it) {
        const unsigned v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if ((unsigned)__builtin_amdgcn_readfirstlane((int)v) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// Broadcast lane Q of each group of four lanes to the group (DPP quad_perm).
template <int Q> __device__ __forceinline__ float quad_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), Q * 0x55, 0xf, 0xf, false));
}

// Rows of T = (I + A)^{-1} for a strictly lower 16 x 16 block A, given -A
// row-major in LDS.  Lane 4j + p returns T[j][4p .. 4p+3].  Row j of T solves
// (I + A^T) y = e_j, upper triangular: once y_s is final (s from 15 down), every
// y_r with r < s takes -A[s][r] y_s.  The coefficients of a step are the same
// for every row j, so each lane reads them with one broadcast 16-byte read, and
// y_s comes from the lane of its quad that holds it.
__device__ __forceinline__ f32x4 unit_lower_inverse16_rows(const float *negA) {
    const int lane = threadIdx.x & 63, j = lane >> 2, p = lane & 3;
    // all coefficient rows first, so the 15 dependent steps do not each wait
    // for an LDS round trip
    f32x4 c[16];
#pragma unroll
    for (int s = 1; s < 16; ++s) c[s] = *reinterpret_cast<const f32x4 *>(negA + s * 16 + 4 * p);
    asm volatile("" ::: "memory");
    f32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (4 * p + e == j) ? 1.f : 0.f;
#define GDN_ROWINV_STEP(s)                                                          \
    {                                                                               \
        const float ys = quad_bcast<(s) / 4>(y[(s) % 4]);                           \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(ys, c[s][e], y[e]); \
    }
    GDN_ROWINV_STEP(15) GDN_ROWINV_STEP(14) GDN_ROWINV_STEP(13) GDN_ROWINV_STEP(12)
    GDN_ROWINV_STEP(11) GDN_ROWINV_STEP(10) GDN_ROWINV_STEP(9) GDN_ROWINV_STEP(8)
    GDN_ROWINV_STEP(7) GDN_ROWINV_STEP(6) GDN_ROWINV_STEP(5) GDN_ROWINV_STEP(4)
    GDN_ROWINV_STEP(3) GDN_ROWINV_STEP(2) GDN_ROWINV_STEP(1)
#undef GDN_ROWINV_STEP
    return y;
}

// Gram blocks of the chunk, 16 x 16 each: block (I, J), J <= I, holds rows t
// of block I and columns s of block J of A (A_ts = beta_t k_t.k_s e^{gamma_t -
// gamma_s}, s < t) and P (P_ts = q_t.k_s e^{gamma_t - gamma_s}, s <= t).  A
// block is computed transposed (k_s . k_t and k_s . q_t: the A operand is k of
// block J, the B operands k and q of block I), so that each lane ends with four
// consecutive columns s of one row t and writes them as one 8-byte piece in
// fragment order.
template <int NKB>
__device__ __forceinline__ void gram_mma(const Frag<__bf16> (&aJ)[NKB], const Frag<__bf16> (&kI)[NKB],
                                         const Frag<__bf16> (&qI)[NKB], f32x4 &aA, f32x4 &aP)
{
    aA = f32x4{0.f, 0.f, 0.f, 0.f};
    aP = aA;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        aA = mma(aA, aJ[kb], kI[kb]);
        aP = mma(aP, aJ[kb], qI[kb]);
    }
}

} // namespace gdn
