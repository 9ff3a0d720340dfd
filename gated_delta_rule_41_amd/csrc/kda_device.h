// kda_device.h -- device helpers shared by the libkda kernels (gfx950 only).
//
// MFMA wrappers, operand fragments and the LDS position permutation used by
// the chunked KDA kernels.  Everything here is written for CDNA4 wave64:
//
//  * v_mfma_f32_16x16x32_bf16 ("k32"): lane l supplies A[m = l%16][k = 8(l/16)+j]
//    and B[k = 8(l/16)+j][n = l%16] for j = 0..7; it receives
//    D[4(l/16)+i][l%16] for i = 0..3 (the accumulator layout).
//  * v_mfma_f32_16x16x16_bf16 ("k16"): A[m][4(l/16)+j], B[4(l/16)+j][n], j=0..3.
//    Its B layout equals the accumulator layout, so a 16x16 accumulator block
//    can be fed back as the B operand of a k16 product without moving data.
//  * fp32 operands use v_mfma_f32_16x16x4_f32: a k32 (k16) step becomes 8 (4)
//    k4 steps, step j taking the j-th element of every lane's fragment.  Any
//    assignment of logical k to (lane group, element) is valid as long as A and
//    B use the same one.
//
// "Accumulator-compatible" k32 fragments: two stacked accumulator blocks (rows
// 0..15 and 16..31 of the contraction index) give lane group qg the logical k
// {4qg..4qg+3, 16+4qg..16+4qg+3}.  Tiles that meet such a B operand are stored
// in LDS with their contraction index permuted inside every 32-block by perm32
// below, so the matching A fragment is again 8 contiguous elements.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace kda {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct V8;
template <> struct V8<bf16> { typedef bf16x8 t; };
template <> struct V8<float> { typedef f32x8 t; };
template <typename T> struct V4;
template <> struct V4<bf16> { typedef bf16x4 t; };
template <> struct V4<float> { typedef f32x4 t; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x4 mma_k32(f32x4 c, bf16x8 a, bf16x8 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k32(f32x4 c, f32x8 a, f32x8 b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4 mma_k16(f32x4 c, bf16x4 a, bf16x4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(f32x4 c, f32x4 a, f32x4 b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
}

// ------------------------------------------------------------ fragments
template <typename T> __device__ __forceinline__ typename V8<T>::t pack8(f32x4 lo, f32x4 hi);
template <> __device__ __forceinline__ bf16x8 pack8<bf16>(f32x4 lo, f32x4 hi) {
    const bf16x4 a = __builtin_convertvector(lo, bf16x4), b = __builtin_convertvector(hi, bf16x4);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <> __device__ __forceinline__ f32x8 pack8<float>(f32x4 lo, f32x4 hi) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) { r[j] = lo[j]; r[j + 4] = hi[j]; }
    return r;
}
template <typename T> __device__ __forceinline__ typename V4<T>::t pack4(f32x4 x);
template <> __device__ __forceinline__ bf16x4 pack4<bf16>(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
template <> __device__ __forceinline__ f32x4 pack4<float>(f32x4 x) { return x; }


// The exact fp32 values of packed bf16 elements, taken from the bit pattern
// (element 2j in the low half of dword j, element 2j+1 in the high half): one
// shift or mask per value.  Written on the integer bits so that the compiler
// does not rebuild each value with a scalar conversion of its own.
__device__ __forceinline__ f32x4 unpack4(bf16x4 x) {
    const u32x2 w = __builtin_bit_cast(u32x2, x);
    f32x4 r;
    r[0] = __uint_as_float(w[0] << 16);
    r[1] = __uint_as_float(w[0] & 0xffff0000u);
    r[2] = __uint_as_float(w[1] << 16);
    r[3] = __uint_as_float(w[1] & 0xffff0000u);
    return r;
}
__device__ __forceinline__ f32x4 unpack4(f32x4 x) { return x; }

// Element j of four rows of four 16-bit values (bf16 bits), as one column
// {r0[j], r1[j], r2[j], r3[j]}: two byte permutes, no conversion.
template <typename V>
__device__ __forceinline__ bf16x4 col4(const V& r0, const V& r1, const V& r2, const V& r3, int j) {
    static_assert(sizeof(V) == 8, "col4: rows of four 16-bit values");
    const u32x2 w0 = __builtin_bit_cast(u32x2, r0), w1 = __builtin_bit_cast(u32x2, r1);
    const u32x2 w2 = __builtin_bit_cast(u32x2, r2), w3 = __builtin_bit_cast(u32x2, r3);
    const unsigned sel = (j & 1) ? 0x07060302u : 0x05040100u;   // the high or the low half of each word
    u32x2 out;
    out[0] = __builtin_amdgcn_perm(w1[j >> 1], w0[j >> 1], sel);
    out[1] = __builtin_amdgcn_perm(w3[j >> 1], w2[j >> 1], sel);
    return __builtin_bit_cast(bf16x4, out);
}

// hi = bf16(x), lo = bf16(x - hi) for N = 2 or 4 values held as N-element
// bf16 vectors (the pair carries ~16 mantissa bits); hi is unpacked from its
// bits as in unpack4.
template <int N>
__device__ __forceinline__ void split_n(const float (&x)[N], __bf16 __attribute__((ext_vector_type(N)))& hi,
                                        __bf16 __attribute__((ext_vector_type(N)))& lo) {
    static_assert(N == 2 || N == 4, "split_n: 2 or 4 values");
    typedef float FV __attribute__((ext_vector_type(N)));
    typedef __bf16 BV __attribute__((ext_vector_type(N)));
    typedef unsigned WV __attribute__((ext_vector_type(N / 2)));
    FV xv;
#pragma unroll
    for (int j = 0; j < N; ++j) xv[j] = x[j];
    hi = __builtin_convertvector(xv, BV);
    const WV w = __builtin_bit_cast(WV, hi);
    FV h;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        h[2 * j] = __uint_as_float(w[j] << 16);
        h[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
    lo = __builtin_convertvector(xv - h, BV);
}

// hi = T(x); lo = T(x - hi) when SPLIT (the pair carries ~16 mantissa bits).
template <typename T, bool SPLIT>
__device__ __forceinline__ void sts4_split(T* hi, T* lo, f32x4 x) {
    const typename V4<T>::t h = pack4<T>(x);
    *reinterpret_cast<typename V4<T>::t*>(hi) = h;
    if constexpr (SPLIT) *reinterpret_cast<typename V4<T>::t*>(lo) = pack4<T>(x - unpack4(h));
}
template <typename T, bool SPLIT>
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, typename V8<T>::t& hi, typename V8<T>::t& lo) {
    if constexpr (SPLIT) {
        const typename V4<T>::t ha = pack4<T>(a), hb = pack4<T>(b);
        hi = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
        lo = pack8<T>(a - unpack4(ha), b - unpack4(hb));
    } else {
        hi = pack8<T>(a, b);
        lo = hi;
    }
}

__device__ __forceinline__ bf16x4 neg4(bf16x4 x) {
    return __builtin_bit_cast(bf16x4, __builtin_bit_cast(u16x4, x) ^ (unsigned short)0x8000);
}
__device__ __forceinline__ f32x4 neg4(f32x4 x) { return -x; }

// 8 contiguous elements from LDS (16-byte aligned for bf16, 32-byte for fp32).
template <typename T> __device__ __forceinline__ typename V8<T>::t lds8(const T* p) {
    return *reinterpret_cast<const typename V8<T>::t*>(p);
}
template <typename T> __device__ __forceinline__ typename V4<T>::t lds4(const T* p) {
    return *reinterpret_cast<const typename V4<T>::t*>(p);
}
template <typename T> __device__ __forceinline__ void sts4(T* p, f32x4 x) {
    *reinterpret_cast<typename V4<T>::t*>(p) = pack4<T>(x);
}
// 4 contiguous elements of type T from LDS, widened to fp32.
template <typename T> __device__ __forceinline__ f32x4 lds4f(const T* p) {
    typename V4<T>::t v = lds4<T>(p);
    f32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = to_f32(v[j]);
    return r;
}

// Position of contraction index k inside its 32-block for tiles that meet an
// accumulator-compatible fragment: logical {16h + 4qg + j} -> 8qg + 4h + j.
__device__ __forceinline__ int perm32(int k) {
    const int kk = k & 31;
    return (k & ~31) | (((kk >> 2) & 3) << 3) | ((kk >> 4) << 2) | (kk & 3);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() is a
// release/acquire fence as well, which waits for every outstanding global load
// of the wave (vmcnt(0)) and so drains register prefetches at each barrier;
// this one waits for the wave's LDS operations and meets the other waves.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sum over the 16 lanes of a DPP row (lanes 16q..16q+15), returned to every
// lane of the row; the butterfly order makes all 16 results bitwise equal.
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    return v;
}

__device__ __forceinline__ float fast_exp(float x) { return __expf(x); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// sigma'(b) = sigma(b) sigma(-b) = e / (1 + e)^2 with e = exp(-|b|): no 1 - sigma(b)
// cancellation for large logits, and no overflow for very negative ones
__device__ __forceinline__ float sigmoid_deriv(float b) {
    const float e = fast_exp(-fabsf(b));
    const float d = 1.f + e;
    return e / (d * d);
}
constexpr float kLog2e = 1.4426950408889634f;

// (I + N)^{-1} for one strictly lower-triangular 16x16 block N (fp32), by the
// identity (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0), with
// fp32 MFMA.  Every matrix X is carried as the accumulator pair (X, X^T): the
// accumulator layout of X is X's k16 B fragment and that of X^T is X's A
// fragment, so no product needs a trip through LDS.
// In: na[j] = N[cl][4qg+j] and nb[j] = N[4qg+j][cl].  Out: T[4qg+i][cl].
__device__ __forceinline__ f32x4 inv_unit_lower16(f32x4 na, f32x4 nb, int qg, int cl) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = (4 * qg + i == cl) ? 1.f : 0.f;
    const f32x4 p2 = mma_k16(z, na, nb);     // N.N
    const f32x4 p2t = mma_k16(z, nb, na);    // N^T.N^T
    const f32x4 p4 = mma_k16(z, p2t, p2);
    const f32x4 p4t = mma_k16(z, p2, p2t);
    const f32x4 p8 = mma_k16(z, p4t, p4);
    const f32x4 y = mma_k16(eye + p4 + p8, p4t, p8);   // (I + P4)(I + P8)
    const f32x4 zz = mma_k16(y, p2t, y);               // (I + P2) Y
    return mma_k16(zz, -na, zz);                       // (I - N) Z
}

// The same inverse with every product taken as three bf16 MFMAs on hi/lo
// operand pairs (hi.hi + lo.hi + hi.lo, ~16 mantissa bits): a k16 bf16 MFMA
// pass is much shorter than the four fp32 k4 MFMAs of a k16 step, and the
// result is rounded to bf16 before it is used as an operand anyway.
__device__ __forceinline__ f32x4 mma3_k16(f32x4 c, f32x4 a, f32x4 b) {
    const bf16x4 ah = pack4<bf16>(a), bh = pack4<bf16>(b);
    const bf16x4 al = pack4<bf16>(a - unpack4(ah)), bl = pack4<bf16>(b - unpack4(bh));
    c = mma_k16(c, ah, bh);
    c = mma_k16(c, al, bh);
    return mma_k16(c, ah, bl);
}
__device__ __forceinline__ f32x4 inv_unit_lower16_x3(f32x4 na, f32x4 nb, int qg, int cl) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = (4 * qg + i == cl) ? 1.f : 0.f;
    const f32x4 p2 = mma3_k16(z, na, nb);
    const f32x4 p2t = mma3_k16(z, nb, na);
    const f32x4 p4 = mma3_k16(z, p2t, p2);
    const f32x4 p4t = mma3_k16(z, p2, p2t);
    const f32x4 p8 = mma3_k16(z, p4t, p4);
    const f32x4 y = mma3_k16(eye + p4 + p8, p4t, p8);
    const f32x4 zz = mma3_k16(y, p2t, y);
    return mma3_k16(zz, -na, zz);
}


// ---------------------------------------------------- global loads/stores
// Loads N consecutive elements of type T (N*sizeof(T) in {8,16,32} bytes)
// and widens them to fp32.
template <typename T, int N> struct GVec {
    float v[N];
};
template <typename T, int N>
__device__ __forceinline__ void gload(float (&dst)[N], const T* __restrict__ src) {
    if constexpr (sizeof(T) == 2) {
        static_assert(N == 4 || N == 8, "bf16 row piece");
        if constexpr (N == 8) {
            u16x8 raw = *reinterpret_cast<const u16x8*>(src);
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = __uint_as_float(((unsigned)raw[j]) << 16);
        } else {
            u16x4 raw = *reinterpret_cast<const u16x4*>(src);
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j] = __uint_as_float(((unsigned)raw[j]) << 16);
        }
    } else {
        static_assert(N % 4 == 0, "fp32 row piece");
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            f32x4 x = *reinterpret_cast<const f32x4*>(src + j);
            dst[j] = x[0]; dst[j + 1] = x[1]; dst[j + 2] = x[2]; dst[j + 3] = x[3];
        }
    }
}


// A row piece of N input elements kept in registers in its storage format
// (bf16 pairs packed two per register), widened to fp32 only when used.
template <typename T, int N> struct RawRow;
template <int N> struct RawRow<bf16, N> {
    typedef unsigned short u16n __attribute__((ext_vector_type(N)));
    u16n x;
    __device__ __forceinline__ void load(const bf16* p) { x = *reinterpret_cast<const u16n*>(p); }
    __device__ __forceinline__ void zero() { x = (u16n)0; }
    // zero unless ok: applied after an unconditional load (of a clamped,
    // in-bounds row), where the values are first needed, so that no branch
    // around the load makes the compiler wait for its data early
    __device__ __forceinline__ void keep(bool ok) { x = ok ? x : (u16n)0; }
    __device__ __forceinline__ float operator[](int j) const { return __uint_as_float(((unsigned)x[j]) << 16); }
    // Hide the value from the optimiser so widened copies made before this
    // point are not kept alive for uses after it.
    __device__ __forceinline__ void fence() { asm volatile("" : "+v"(x)); }
};
template <int N> struct RawRow<float, N> {
    typedef float fn __attribute__((ext_vector_type(N)));
    fn x;
    __device__ __forceinline__ void load(const float* p) { x = *reinterpret_cast<const fn*>(p); }
    __device__ __forceinline__ void zero() { x = (fn)0.f; }
    __device__ __forceinline__ void keep(bool ok) { x = ok ? x : (fn)0.f; }
    __device__ __forceinline__ float operator[](int j) const { return x[j]; }
    __device__ __forceinline__ void fence() { asm volatile("" : "+v"(x)); }
};

// One input scalar kept in storage format until used.
template <typename T> struct RawScalar;
template <> struct RawScalar<bf16> {
    unsigned short x;
    __device__ __forceinline__ void load(const bf16* p) { x = *reinterpret_cast<const unsigned short*>(p); }
    __device__ __forceinline__ void zero() { x = 0; }
    __device__ __forceinline__ float f() const { return __uint_as_float(((unsigned)x) << 16); }
};
template <> struct RawScalar<float> {
    float x;
    __device__ __forceinline__ void load(const float* p) { x = *p; }
    __device__ __forceinline__ void zero() { x = 0.f; }
    __device__ __forceinline__ float f() const { return x; }
};

// Element `idx` of an array whose base is uniform across the wave, addressed
// with a 32-bit byte offset (idx * sizeof(E) < 2^32): lets the compiler use
// the scalar-base + 32-bit vector offset form of global loads and stores
// instead of a 64-bit address add per access.
template <typename E>
__device__ __forceinline__ E* atb(E* base, unsigned byte_off) {
    typedef typename std::conditional<std::is_const<E>::value, const char, char>::type C;
    return reinterpret_cast<E*>(reinterpret_cast<C*>(base) + byte_off);
}
template <typename E>
__device__ __forceinline__ E* at32(E* base, unsigned idx) { return atb(base, idx * (unsigned)sizeof(E)); }

template <typename T> __device__ __forceinline__ float gload1(const T* p) { return to_f32(*p); }

template <typename T> __device__ __forceinline__ void gstore1(T* p, float x) { *p = from_f32<T>(x); }

// ------------------------------------------------------- work mapping
// Block -> (chain, slice).  Slices of one chain get block ids b and b+8, which
// the dispatcher places on the same XCD, so their duplicate q/k/g reads share
// that XCD's L2.
__device__ __forceinline__ void map_block(int b, int nchains, int ns, int& chain, int& slice) {
    const int total = nchains * ns;
    if (ns > 1 && (total % (8 * ns)) == 0) {
        const int x = b & 7, r = b >> 3;
        slice = r % ns;
        chain = (r / ns) * 8 + x;
    } else {
        chain = b / ns;
        slice = b % ns;
    }
}

__device__ __forceinline__ void seq_bounds(const int32_t* cu, int n, int seqlen, int64_t T,
                                           int64_t& t0, int64_t& t1) {
    if (cu) {
        int64_t a = cu[n], z = cu[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        z = z < a ? a : (z > T ? T : z);
        t0 = a;
        t1 = z;
    } else {
        t0 = (int64_t)n * seqlen;
        t1 = t0 + seqlen;
    }
}

// acc += A.B with optional hi/lo operands: Ah.Bh + Ah.Bl + Al.Bh.
template <bool SPLIT, typename V>
__device__ __forceinline__ f32x4 mma3(f32x4 acc, const V& ah, const V& al, const V& bh, const V& bl) {
    acc = mma_k32(acc, ah, bh);
    if constexpr (SPLIT) {
        acc = mma_k32(acc, ah, bl);
        acc = mma_k32(acc, al, bh);
    }
    return acc;
}

}  // namespace kda
