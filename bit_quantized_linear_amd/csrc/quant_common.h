// Device helpers shared by the activation quantizers (the standalone pass in
// act_quant.hip and the fused MLP epilogue of the FP6 GEMM): exact fp32
// quotients without per-element divisions, the FP6 E2M3 field of an INT4
// code, and the packing of codes into FP6 fields by the conversion
// instruction.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"

namespace svdq {

// Groups whose largest |x / s| is below this take IEEE divisions (see
// quotient_fp32).
constexpr float kTinyGroup = 0x1p-100f;

// fp32(a / b), correctly rounded, from r = fp64(1 / b) (correctly rounded):
// d = fp64(a * r) is within 2^-52 (relative) of a / b. A quotient of two
// fp32 values with 24-bit significands lies either exactly on an fp32 value
// or at least 2^-49 (relative) away from every fp32 rounding boundary (a
// midpoint has an odd 25-bit significand; a / b equal to or within 2^-49 of
// one would need a 49-bit numerator), so d and a / b round to the same fp32
// value. This holds while the result is a normal fp32 number or overflows;
// results below 2^-126 can fall on a subnormal midpoint, which the caller
// excludes (groups whose largest |x / s| is below 2^-100 use IEEE division,
// and in any other group a subnormal x / s becomes code 0 whatever its
// exact value, as it is below 7 * 2^-26 of the scale).
__device__ __forceinline__ float quotient_fp32(float a, double r) {
    return (float)((double)a * r);
}

// INT4 code of x_hat for a group scale with reciprocal rscale = fp64(1 /
// scale): round half to even of the exact fp32 quotient, clamped to [-7, 7].
__device__ __forceinline__ int int4_code(float xh, double rscale) {
    const float q = rintf(quotient_fp32(xh, rscale));
    return (int)fminf(7.0f, fmaxf(-7.0f, q));
}

// FP6 E2M3 field of code c in [-7, 7] as the value c / 8: sign bit 5, zero
// exponent, magnitude in the 3 mantissa bits.
__device__ __forceinline__ uint32_t fp6_field(int c) {
    return (c < 0 ? 0x20u : 0u) | (uint32_t)(c < 0 ? -c : c);
}

// 1/7 rounded to fp64, for the group scale amax / 7.
constexpr double kRcp7 = 1.0 / 7.0;

// The FP6 E2M3 value c / 8 of code c = clamp(RNE(fp32(x_hat / scale)), -7,
// 7), with +0 for a zero code (the fma adds +0, which turns -0 into +0 and
// leaves every other value as it is).
__device__ __forceinline__ float fp6_value(float xh, double rscale) {
    const float c = fminf(7.0f, fmaxf(-7.0f, rintf(quotient_fp32(xh, rscale))));
    return __builtin_fmaf(c, 0.125f, 0.0f);
}

// FP6 E2M3 fields of v[0..15] (values that are exactly representable),
// packed LSB-first into 3 dwords. The conversion interleaves its two
// 16-value operands field by field (first[0], second[0], first[1], ...), so
// even-indexed values go in the first and odd-indexed ones in the second;
// their upper halves would fill three more dwords, which are not used.
__device__ __forceinline__ void pack_fp6_16(const float (&v)[16], uint32_t (&w)[3]) {
    // the upper halves are left undefined, so that no register is spent or
    // copied for them (the compiler may overlap the two operands)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wuninitialized"
    f32x16 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = v[2 * i];
        b[i] = v[2 * i + 1];
    }
    auto r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
    // Both operands stay live until after the conversion (an empty asm
    // statement that reads them and passes the result through, so it cannot
    // move above the conversion): its result is then never given registers
    // of an operand. With the result starting on the second operand's third
    // register (v[16:21] over v[14:29]) the instruction packed a 0 for that
    // value.
    asm volatile("" : "+v"(r) : "v"(a), "v"(b));
#pragma clang diagnostic pop
    w[0] = r[0];
    w[1] = r[1];
    w[2] = r[2];
}

}  // namespace svdq
