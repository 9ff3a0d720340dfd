// kda_f16.h -- fp16 matrix-core helpers shared by the bf16-input kernels that
// use single-rounding fp16 operands (kda_fwd16.hip, kda_scan16.hip).
//
//  * v_mfma_f32_16x16x32_f16 ("mma32"): lane (qg, cl) supplies A[m = cl][k =
//    8qg + j] and B[k = 8qg + j][n = cl], j < 8, and receives D[4qg + i][cl].
//  * v_mfma_f32_16x16x16_f16 ("mma16"): A[m = cl][k = 4qg + j], B[4qg + j][cl];
//    its B layout is the accumulator layout.
#pragma once
#include "kda_device.h"

namespace kda {
namespace f16 {

typedef _Float16 h16;
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 hx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mma32(f32x4 c, h8 a, h8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 c, h4 a, h4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ h4 cvt4(f32x4 x) { return __builtin_convertvector(x, h4); }
__device__ __forceinline__ h8 cvt8(f32x4 a, f32x4 b) {
    const h4 x = cvt4(a), y = cvt4(b);
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <int N>
__device__ __forceinline__ void cvt_store(h16* dst, const float (&x)[N]) {
    typedef float FV __attribute__((ext_vector_type(N)));
    typedef _Float16 HV __attribute__((ext_vector_type(N)));
    FV v;
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = x[j];
    *reinterpret_cast<HV*>(dst) = __builtin_convertvector(v, HV);
}

// Wave-wide maximum of non-negative values, as a wave-uniform value: DPP
// within each 16-lane row, then the four row results.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v));   // row_mirror
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
// Sum over the four lanes that share l % 16 (l, l^16, l^32, l^48): every one
// of them gets the same bits.
__device__ __forceinline__ float qsum(float v) {
    v += __shfl_xor(v, 16);
    return v + __shfl_xor(v, 32);
}

// U and dU of a chunk (fp16, per head [64 tokens][dv]) are stored in MFMA
// fragment order: 16-column group g = j >> 4, then row block ib = t >> 4, then
// the accumulator lane (qg = (t >> 2) & 3, cl = j & 15), then i = t & 3, so that
// the 16x16 block a wave holds in an accumulator is 512 contiguous bytes.
__host__ __device__ constexpr int ufrag(int t, int j) {
    return (((j >> 4) * 4 + (t >> 4)) * 64 + ((t >> 2) & 3) * 16 + (j & 15)) * 4 + (t & 3);
}

constexpr float kUnsafe = -14.f;   // lowest per-block log2 decay the fp16 factors hold


// A 16x16 fp32 block in the accumulator layout (lane (qg, cl): rows 4qg + i,
// column cl) as fp16 rows: the block enters the matrix core as the A operand
// against an identity B (eye[j] = (4qg + j == cl)), which hands lane (qg, cl)
// row cl, columns 4qg .. 4qg + 3 -- four consecutive elements for one store.
// Exact: fp16 values times one.
__device__ __forceinline__ h4 block_rows4(f32x4 x, h4 eye) {
    return cvt4(mma16(f32x4{0.f, 0.f, 0.f, 0.f}, cvt4(x), eye));
}
__device__ __forceinline__ h4 block_eye4(int qg, int cl) {
    h4 e;
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = (h16)((4 * qg + j == cl) ? 1.f : 0.f);
    return e;
}

// Four 16-bit values through the LDS transpose read (ds_read_b64_tr_b16): every
// lane names 8 bytes, and inside each row of 16 lanes lane t receives element
// (t & 3) of the 8 bytes named by lanes 4k + (t >> 2), k = 0..3 (the layout as
// measured on gfx950).  A row-major [r][c] tile read with lane l of a row naming
// (r0 + (l >> 2), c0 + 4 (l & 3)) gives lane t the column c0 + t, rows r0..r0+3.
__device__ __forceinline__ h4 lds_tr4(const h16* p) {
    typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(const_cast<h16*>(p)));
    return __builtin_bit_cast(h4, r);
}

// r * stride + add as a 32-bit VGPR offset.  The multiply is kept apart from the
// add: fused, the compiler emits a 64-bit multiply-add whose unused upper addend
// half can be a register a load in flight still targets, and then waits for that
// load before issuing the next ones.
__device__ __forceinline__ unsigned row_off(int r, int stride, int add) {
    unsigned m = (unsigned)r * (unsigned)stride;
    asm volatile("" : "+v"(m));
    return m + (unsigned)add;
}

}  // namespace f16
}  // namespace kda
