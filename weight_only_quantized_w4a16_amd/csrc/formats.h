// The 8-bit activation and weight formats of libqgemm's W8A8 and W4A8 paths
// (device side): the code map, q_max, the k-tile product and the accumulator
// type of each, and the code quotient of the quantization fused into a GEMM.
#pragma once

#include "device_common.h"

namespace qg {

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct FmtE4M3 {
    static constexpr float qmax = 448.0f;
    using acc_t = f32x4;
    using elem_t = float;
    // two fp32 quotients -> two codes (low byte = first value)
    __device__ static __forceinline__ uint32_t encode2(float a, float b) {
        a = fminf(fmaxf(a, -448.0f), 448.0f);
        b = fminf(fmaxf(b, -448.0f), 448.0f);
        return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
    }
    // acc + A . B over one 128-deep k-tile; a0/b0 hold k = 16*(lane/16) + 0..15,
    // a1/b1 the same 64 rows further
    __device__ static __forceinline__ acc_t mma(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, acc_t c) {
        return mfma_fp8_16x16x128(cat_i32x8(a0, a1), cat_i32x8(b0, b1), c);
    }
    __device__ static __forceinline__ acc_t zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ static __forceinline__ float value(elem_t x) { return x; }
};

struct FmtI8 {
    static constexpr float qmax = 127.0f;
    using acc_t = i32x4;
    using elem_t = int;
    __device__ static __forceinline__ uint32_t encode2(float a, float b) {
        const int qa = (int)fminf(fmaxf(rintf(a), -127.0f), 127.0f);   // half to even
        const int qb = (int)fminf(fmaxf(rintf(b), -127.0f), 127.0f);
        return ((uint32_t)qa & 0xffu) | (((uint32_t)qb & 0xffu) << 8);
    }
    __device__ static __forceinline__ acc_t mma(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, acc_t c) {
        c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a0),
                                                  __builtin_bit_cast(i32x4, b0), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a1),
                                                     __builtin_bit_cast(i32x4, b1), c, 0, 0, 0);
    }
    __device__ static __forceinline__ acc_t zero() { return i32x4{0, 0, 0, 0}; }
    __device__ static __forceinline__ float value(elem_t x) { return (float)x; }
};

// Quotient a / s whose code the fused per-token quantization takes: with
// r = 1/s (IEEE), q0 = a r, e = fma(-q0, s, a), q = fma(e, r, q0) -- one
// correction step of the reciprocal product, three operations instead of a
// full division.  It can differ from the IEEE quotient in its last bit but
// never in the code it rounds to, for every pair of bf16 values |a| <= amax
// with s = amax / q_max >= 2^-100 in both formats (an exhaustive check over
// all such pairs); `fast` is false for smaller or non-finite scales, which
// divide.
template <class Fmt>
__device__ __forceinline__ float dyn_quotient(float x, float s, float r, bool fast) {
    if (!fast) return x / s;
    const float q0 = x * r;
    const float e = fmaf(-q0, s, x);
    return fmaf(e, r, q0);
}

}  // namespace qg
