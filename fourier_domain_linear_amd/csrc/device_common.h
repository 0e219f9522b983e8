// device_common.h -- small gfx950 helpers shared by the library's kernels: bf16 / fp16 packing and the
// half-precision matrix-core instructions used by the spectral and expanded kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dft.h"

namespace eqlin {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float bf16_at(const uint4 &v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// 8 fp32 -> 8 bf16 (round to nearest even; gfx950 has a packed hardware conversion for this).
__device__ __forceinline__ uint4 pack_bf16x8(const float *f) {
    f32x8 v = {f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
    bf16x8 h = __builtin_convertvector(v, bf16x8);
    return __builtin_bit_cast(uint4, h);
}

// 2 fp32 -> one word of 2 bf16 (RNE), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t pack_bf16(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// Flip the sign of 8 packed bf16 values.
__device__ __forceinline__ uint4 neg_bf16x8(const uint4 &v) {
    return make_uint4(v.x ^ 0x80008000u, v.y ^ 0x80008000u, v.z ^ 0x80008000u, v.w ^ 0x80008000u);
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Operand layout (lane l of 64): A row l%16, B column l%16, both holding the 8 consecutive k values
// 8*(l/16) .. 8*(l/16)+7; D: lane l holds rows 4*(l/16) + v (v = 0..3) of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(const uint4 &a, const uint4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Operand layout (lane l of 64): A row l%32, B column l%32, both holding the 8 consecutive k values
// 8*(l/32) .. 8*(l/32)+7; D: lane l holds rows 8*(v/4) + 4*(l/32) + v%4 (v = 0..15) of column l%32.
__device__ __forceinline__ f32x16 mfma32x32x16(const uint4 &a, const uint4 &b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- Element types. The half-precision paths run in bf16 (the default) or IEEE fp16 (the page's FP16
// kernels, "Implementación"); kernels take one of these tags and use the helpers below, which for
// BF16 are exactly the bf16 functions above. ----
struct BF16 {
    static constexpr uint32_t kOne = 0x3f80u;  // 1.0
};
struct F16 {
    static constexpr uint32_t kOne = 0x3c00u;  // 1.0
};
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <class E>
__device__ __forceinline__ float elem_lo(uint32_t w) {
    if constexpr (__is_same(E, F16)) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    else return bf16_lo(w);
}
template <class E>
__device__ __forceinline__ float elem_hi(uint32_t w) {
    if constexpr (__is_same(E, F16)) return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    else return bf16_hi(w);
}
template <class E>
__device__ __forceinline__ float elem_at(const uint4 &v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? elem_hi<E>(w) : elem_lo<E>(w);
}
template <class E>
__device__ __forceinline__ float elem_to_float(uint16_t bits) { return elem_lo<E>(bits); }
// 8 fp32 -> 8 elements, round to nearest even
template <class E>
__device__ __forceinline__ uint4 pack8(const float *f) {
    if constexpr (__is_same(E, F16)) {
        f32x8 v = {f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]};
        return __builtin_bit_cast(uint4, __builtin_convertvector(v, f16x8));
    } else {
        return pack_bf16x8(f);
    }
}
template <class E>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (__is_same(E, F16)) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        f32x2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    } else {
        return pack_bf16x2(a, b);
    }
}
template <class E>
__device__ __forceinline__ uint16_t pack1(float a) {
    if constexpr (__is_same(E, F16)) return __builtin_bit_cast(uint16_t, (_Float16)a);
    else return pack_bf16(a);
}
// the matrix-core products of mfma16x16x32 / mfma32x32x16 in the element type (same layouts)
template <class E>
__device__ __forceinline__ f32x4 mma16(const uint4 &a, const uint4 &b, f32x4 c) {
    if constexpr (__is_same(E, F16))
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return mfma16x16x32(a, b, c);
}
template <class E>
__device__ __forceinline__ f32x16 mma32(const uint4 &a, const uint4 &b, f32x16 c) {
    if constexpr (__is_same(E, F16))
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return mfma32x32x16(a, b, c);
}
// neg_bf16x8 flips the sign bit of each 16-bit lane: the same for fp16.

// Number of real matrix products per frequency-plane set (k = 0 and G/2 real, the rest complex).
__host__ __device__ constexpr int real_products(int G) { return G == 1 ? 1 : 2 * G - 2; }

}  // namespace eqlin
