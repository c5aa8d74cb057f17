// Device helpers shared by the activation quantizers (the standalone pass in
// act_quant.hip and the fused MLP epilogue of the FP6 GEMM): exact fp32
// quotients without per-element divisions, and the FP6 E2M3 field of an
// INT4 code.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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

}  // namespace svdq
