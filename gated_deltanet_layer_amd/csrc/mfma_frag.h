// mfma_frag.h -- MFMA operand fragments for the chunkwise kernels (gfx950).
//
// A fragment is one lane's share of a 16 x 32 operand (16 rows, 32 k values),
// in the k-slot order described in gdn_common.h: lane group gq supplies the k
// columns k0 + 4*gq .. +3 and k0 + 16 + 4*gq .. +3.  An accumulator tile
// (rows 4*gq + e of column r16) therefore feeds the next product as its B
// operand without any data movement (reg_frag).
#pragma once
#include "gdn_common.h"

namespace gdn {

template <typename OT> struct Frag;
template <> struct Frag<__bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ int lane_r16() { return threadIdx.x & 15; }
__device__ __forceinline__ int lane_gq() { return (threadIdx.x & 63) >> 4; }

// Row-major matrix M in LDS; fragment rows row0 .. row0+15, k columns
// k0 + 4*gq .. +3 and k0 + 16 + 4*gq .. +3 for lane group gq.
__device__ __forceinline__ Frag<__bf16> lds_frag(const __bf16 *M, int ld, int row0, int k0) {
    const __bf16 *p = M + (row0 + lane_r16()) * ld + k0 + 4 * lane_gq();
    return {cat8(*reinterpret_cast<const bf16x4 *>(p), *reinterpret_cast<const bf16x4 *>(p + 16))};
}
__device__ __forceinline__ Frag<float> lds_frag(const float *M, int ld, int row0, int k0) {
    const float *p = M + (row0 + lane_r16()) * ld + k0 + 4 * lane_gq();
    return {*reinterpret_cast<const f32x4 *>(p), *reinterpret_cast<const f32x4 *>(p + 16)};
}
// Same, with only the first 16 k columns; the other half is zero.
__device__ __forceinline__ Frag<__bf16> lds_frag_lo(const __bf16 *M, int ld, int row0, int k0) {
    const __bf16 *p = M + (row0 + lane_r16()) * ld + k0 + 4 * lane_gq();
    const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    return {cat8(*reinterpret_cast<const bf16x4 *>(p), z)};
}
__device__ __forceinline__ Frag<float> lds_frag_lo(const float *M, int ld, int row0, int k0) {
    const float *p = M + (row0 + lane_r16()) * ld + k0 + 4 * lane_gq();
    return {*reinterpret_cast<const f32x4 *>(p), f32x4{0.f, 0.f, 0.f, 0.f}};
}

// K^T staging is swizzled: the 16 column groups of 4 tokens are permuted per
// channel row, so that both the packed transposed writes (one lane per group of
// EPV channels) and the fragment reads (16 consecutive channel rows per lane
// group) hit distinct LDS banks.  kmt_swz(c) is a multiple of 4 below 64.
template <int EPV> __device__ __forceinline__ int kmt_swz(int c) {
    return (((c / EPV) ^ ((c % EPV) * (16 / EPV))) & 15) << 2;
}

template <int EPV>
__device__ __forceinline__ Frag<__bf16> lds_frag_kmt(const __bf16 *M, int ld, int row0, int k0) {
    const int c = row0 + lane_r16(), s = kmt_swz<EPV>(c), col = k0 + 4 * lane_gq();
    const __bf16 *p = M + c * ld;
    return {cat8(*reinterpret_cast<const bf16x4 *>(p + (col ^ s)),
                 *reinterpret_cast<const bf16x4 *>(p + ((col + 16) ^ s)))};
}
template <int EPV>
__device__ __forceinline__ Frag<float> lds_frag_kmt(const float *M, int ld, int row0, int k0) {
    const int c = row0 + lane_r16(), s = kmt_swz<EPV>(c), col = k0 + 4 * lane_gq();
    const float *p = M + c * ld;
    return {*reinterpret_cast<const f32x4 *>(p + (col ^ s)),
            *reinterpret_cast<const f32x4 *>(p + ((col + 16) ^ s))};
}

// Fragment-ordered storage ("frag order"): inside each block of 32 columns the
// columns are stored in the order lane group gq reads them, so one lane's
// fragment (logical columns k0 + 4gq .. +3 and k0 + 16 + 4gq .. +3) is 16
// contiguous bytes and loads with one 16-byte LDS read.  Groups of 4
// consecutive logical columns stay contiguous.
__device__ __forceinline__ constexpr int frag_col(int c) {
    return (c & ~31) | (((c & 15) >> 2) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}
__device__ __forceinline__ Frag<__bf16> lds_frag_fo(const __bf16 *M, int ld, int row0, int k0) {
    return {*reinterpret_cast<const bf16x8 *>(M + (row0 + lane_r16()) * ld + k0 + 8 * lane_gq())};
}
// First 16 logical columns only (the other half zero).
__device__ __forceinline__ Frag<__bf16> lds_frag_fo_lo(const __bf16 *M, int ld, int row0, int k0) {
    const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    return {cat8(*reinterpret_cast<const bf16x4 *>(M + (row0 + lane_r16()) * ld + k0 + 8 * lane_gq()), z)};
}

// Unpadded fragment-order rows with their 16-byte chunks XOR-swizzled per row
// (chunk ^ swz), so the 16 rows of a fragment read fall on distinct banks.
// swz is a chunk count below the number of chunks in a row; groups of 4
// columns stay contiguous.
__device__ __forceinline__ Frag<__bf16> lds_frag_fos(const __bf16 *M, int ld, int row0, int k0,
                                                    int swz) {
    return {*reinterpret_cast<const bf16x8 *>(M + (row0 + lane_r16()) * ld +
                                              ((k0 + 8 * lane_gq()) ^ (swz << 3)))};
}

// B operand from two accumulator tiles holding rows k0..k0+15 and k0+16..k0+31.
template <typename OT> __device__ __forceinline__ Frag<OT> reg_frag(f32x4 c0, f32x4 c1);
template <> __device__ __forceinline__ Frag<__bf16> reg_frag<__bf16>(f32x4 c0, f32x4 c1) {
    return {cat8(cvt4(c0), cvt4(c1))};
}
template <> __device__ __forceinline__ Frag<float> reg_frag<float>(f32x4 c0, f32x4 c1) {
    return {c0, c1};
}

__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<__bf16> &a, const Frag<__bf16> &b) {
    return mfma_bf16(a.v, b.v, acc);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32(a.lo[e], b.lo[e], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32(a.hi[e], b.hi[e], acc);
    return acc;
}
// Product over the first 16 k only (a's upper half is zero).
__device__ __forceinline__ f32x4 mma_lo(f32x4 acc, const Frag<__bf16> &a, const Frag<__bf16> &b) {
    return mfma_bf16(a.v, b.v, acc);
}
__device__ __forceinline__ f32x4 mma_lo(f32x4 acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mfma_f32(a.lo[e], b.lo[e], acc);
    return acc;
}

// Multiply the k-slots of a fragment by per-column factors f[k] (f in LDS).
__device__ __forceinline__ Frag<__bf16> scale_frag(Frag<__bf16> x, const float *f, int k0) {
    const int gq = lane_gq();
    const f32x4 f0 = *reinterpret_cast<const f32x4 *>(f + k0 + 4 * gq);
    const f32x4 f1 = *reinterpret_cast<const f32x4 *>(f + k0 + 16 + 4 * gq);
    f32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (float)x.v[e] * f0[e];
        b[e] = (float)x.v[4 + e] * f1[e];
    }
    return {cat8(cvt4(a), cvt4(b))};
}
__device__ __forceinline__ Frag<float> scale_frag(Frag<float> x, const float *f, int k0) {
    const int gq = lane_gq();
    const f32x4 f0 = *reinterpret_cast<const f32x4 *>(f + k0 + 4 * gq);
    const f32x4 f1 = *reinterpret_cast<const f32x4 *>(f + k0 + 16 + 4 * gq);
    return {x.lo * f0, x.hi * f1};
}

// Packs of N elements of type T (for the transposed K writes).
template <typename T, int N> struct Pack;
template <> struct Pack<__bf16, 4> { typedef bf16x4 type; };
template <> struct Pack<__bf16, 2> { typedef bf16x2 type; };
template <> struct Pack<float, 4> { typedef f32x4 type; };


// Gram blocks (i, j), j <= i, handled by wave w (0..3) in step pp (0..2):
//   w0: (3,0) (3,1) (0,0)   w1: (3,2) (3,3)   w2: (2,0) (2,1) (2,2)   w3: (1,0) (1,1)
// Rows are grouped so a wave reuses its left-hand fragments, and every wave owns
// exactly one diagonal block.  i < 0 marks an empty step.  w must be
// wave-uniform; the selection compiles to scalar instructions.
__device__ __forceinline__ void gram_block(int w, int pp, int &i, int &j) {
    if (w == 0) { i = pp < 2 ? 3 : 0; j = pp < 2 ? pp : 0; }
    else if (w == 1) { i = pp < 2 ? 3 : -1; j = pp + 2; }
    else if (w == 2) { i = 2; j = pp; }
    else { i = pp < 2 ? 1 : -1; j = pp; }
}

} // namespace gdn
