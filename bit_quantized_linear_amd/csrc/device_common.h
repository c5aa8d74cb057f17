// Device-side helpers for the gfx950 (CDNA4) kernels of libsvdq.so:
// vector types, MFMA wrappers and the fixed rounding points.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svdq {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- MFMA (gfx950) ---------------------------------------------------------
// 32x32 outputs: lane l holds column (l % 32) and rows 8q + 4(l / 32) + t at
// element 4q + t (q, t in 0..3). 16x16 outputs: lane l holds column (l % 16)
// and rows 4(l / 16) + t at element t. A lane's A operand is one row and its
// B operand one column; A and B lanes of the same lane index carry the same
// K slots, so any K permutation applied identically to both leaves the
// product unchanged.

__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b, i32x16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- conversions -----------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 -> packed bf16 (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950. Same result as f32_to_bf16_bits for every
// non-NaN input.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <class T>
__device__ __forceinline__ T bitcast(const void *p) {
    return *reinterpret_cast<const T *>(p);
}

// Nibble unpack for the INT4 path: 8 packed bytes (16 two's-complement
// nibbles, low nibble = even k) become 16 int8 values equal to 16 * code, in
// the order [k0, k2, ..., k14, k1, k3, ..., k15]. Shifting a nibble into the
// high half of its byte multiplies it by 16 exactly; the factor 16 * 16 = 256
// of a product is removed after the integer sum, exactly.
__device__ __forceinline__ void unpack_int4x16(uint32_t a, uint32_t b, uint32_t out[4]) {
    out[0] = (a << 4) & 0xF0F0F0F0u;
    out[1] = (b << 4) & 0xF0F0F0F0u;
    out[2] = a & 0xF0F0F0F0u;
    out[3] = b & 0xF0F0F0F0u;
}

}  // namespace svdq
