// gdn_common.h -- small device helpers shared by the gfx950 kernels.
//
// MFMA operand layout used throughout (CDNA3/CDNA4 matrix cores, wave64):
//   lane l = 16 * gq + r  (gq = l / 16 in 0..3, r = l % 16)
//   C/D tile 16x16 fp32:  lane holds rows 4*gq + {0,1,2,3} of column r.
//   A operand:            lane holds row r, a run of k-slots chosen by gq.
//   B operand:            lane holds column r, the same run of k-slots.
// Because A and B use the same k-slots per lane group, any fixed bijection
// between k-slots and the contraction index works, provided A and B agree.
// We use the one that lets a C tile feed the next product as its B operand
// without moving data between lanes: for a 32-wide k block made of two
// 16-row slabs s0, s1, lane group gq supplies rows
//   {16*s0 + 4*gq + i, 16*s1 + 4*gq + i : i = 0..3}
// (bf16 16x16x32), and for fp32 16x16x4 the k-step j uses row 4*gq + j of the
// slab.  An A operand read from LDS must then take, for its row r, the four
// contiguous columns 16*s + 4*gq .. +3 of each slab.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ bf16x4 cvt4(f32x4 v) {
    bf16x4 r;
    r[0] = (__bf16)v[0];
    r[1] = (__bf16)v[1];
    r[2] = (__bf16)v[2];
    r[3] = (__bf16)v[3];
    return r;
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc += A(16x32) * B(32x16), bf16 operands, fp32 accumulate.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// acc += A(16x4) * B(4x16), fp32 operands.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also fences global
// memory, which waits for every outstanding global load and store of the wave;
// the kernels keep prefetches and output stores in flight across barriers, so
// they wait only for LDS operations (lgkmcnt) before s_barrier.  The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP shifts within each
// row of 16 lanes, then the row totals are added with readlane.
template <int CTRL> __device__ __forceinline__ float dpp_shr(float x) {
    // row_shr:n with bound_ctrl: lanes without a source read 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_shr<0x111>(x);   // row_shr:1
    x += dpp_shr<0x112>(x);   // row_shr:2
    x += dpp_shr<0x114>(x);   // row_shr:4
    x += dpp_shr<0x118>(x);   // row_shr:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
    const int row = (threadIdx.x & 63) >> 4;
    const float off = row == 0 ? 0.f : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2;
    return x + off;
}

// Broadcast 16-lane row R of x to all four rows of the wave (gfx950 permlane
// swaps: the 16-lane swap exchanges odd rows of one operand with even rows of
// the other, the 32-lane swap the upper half of one with the lower half of the
// other).
template <int R> __device__ __forceinline__ float row_broadcast(float x) {
    const int xi = __float_as_int(x);
    const auto s16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
    const int a = (R & 1) ? (int)s16[1] : (int)s16[0];      // rows {R%2, R%2, R%2+2, R%2+2}
    const auto s32 = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    return __int_as_float((R & 2) ? (int)s32[1] : (int)s32[0]);
}

// Broadcast lane N of each 16-lane row to the whole row (DPP row_newbcast).
template <int N> __device__ __forceinline__ float lane_in_row(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xf, 0xf, false));
}

// Inverse of a unit lower triangular 16 x 16 matrix I + A held in the MFMA
// accumulator layout (lane 16*gq + j holds A[4gq + e][j], e = 0..3; A strictly
// lower).  Returns T = (I + A)^{-1} in the same layout.  Column j is built by
// forward substitution, right-looking: once row r is final, every later row
// subtracts A[row][r] * T[r][j].  The pivot row comes from one lane group
// (row_broadcast), the column of A from one lane of each row (lane_in_row);
// A's zeros on and above the diagonal make the update a no-op where it must be.
__device__ __forceinline__ f32x4 unit_lower_inverse16(f32x4 a) {
    const int lane = threadIdx.x & 63, gq = lane >> 4, j = lane & 15;
    f32x4 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (4 * gq + e == j) ? 1.f : 0.f;
#define GDN_INV_STEP(r)                                                   \
    {                                                                     \
        const float piv = row_broadcast<(r) / 4>(t[(r) % 4]);             \
        _Pragma("unroll") for (int e = 0; e < 4; ++e)                     \
            t[e] -= lane_in_row<(r)>(a[e]) * piv;                         \
    }
    GDN_INV_STEP(0) GDN_INV_STEP(1) GDN_INV_STEP(2) GDN_INV_STEP(3)
    GDN_INV_STEP(4) GDN_INV_STEP(5) GDN_INV_STEP(6) GDN_INV_STEP(7)
    GDN_INV_STEP(8) GDN_INV_STEP(9) GDN_INV_STEP(10) GDN_INV_STEP(11)
    GDN_INV_STEP(12) GDN_INV_STEP(13) GDN_INV_STEP(14)
#undef GDN_INV_STEP
    return t;
}

// Inverse of a unit upper triangular 16 x 16 matrix I + U held in the MFMA
// accumulator layout (lane 16*gq + j holds U[4gq + e][j]; U strictly upper).
// Returns (I + U)^{-1} in the same layout, by backward substitution:
// once row r is final, every earlier row subtracts U[row][r] * X[r][j].
__device__ __forceinline__ f32x4 unit_upper_inverse16(f32x4 u) {
    const int lane = threadIdx.x & 63, gq = lane >> 4, j = lane & 15;
    f32x4 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = (4 * gq + e == j) ? 1.f : 0.f;
#define GDN_INVU_STEP(r)                                                  \
    {                                                                     \
        const float piv = row_broadcast<(r) / 4>(t[(r) % 4]);             \
        _Pragma("unroll") for (int e = 0; e < 4; ++e)                     \
            t[e] -= lane_in_row<(r)>(u[e]) * piv;                         \
    }
    GDN_INVU_STEP(15) GDN_INVU_STEP(14) GDN_INVU_STEP(13) GDN_INVU_STEP(12)
    GDN_INVU_STEP(11) GDN_INVU_STEP(10) GDN_INVU_STEP(9) GDN_INVU_STEP(8)
    GDN_INVU_STEP(7) GDN_INVU_STEP(6) GDN_INVU_STEP(5) GDN_INVU_STEP(4)
    GDN_INVU_STEP(3) GDN_INVU_STEP(2) GDN_INVU_STEP(1)
#undef GDN_INVU_STEP
    return t;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

} // namespace gdn
