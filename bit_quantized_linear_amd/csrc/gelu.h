// bf16(GELU(y)) of a bf16 value y with one correct rounding of the exact
// GELU(y) = y Phi(y) = (y / 2) erfc(-y / sqrt 2), the activation between the
// two projections of a DiT MLP.
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
// and "Nunchaku Lite" paragraphs (svdq_w4a4 on the MLP projections, fused
// kernels); the erf form of GELU is the DiT MLP's.
//
// y takes only 2^16 values, so the rounding is decided exactly:
//  * 2^-9 <= |y| < 16: a table (gelu_table.h, generated at build time from
//    float64 erfc with a checked error margin), held in LDS by the caller;
//  * 2^-125 <= |y| < 2^-9: y / 2, exactly. GELU(y) = (y / 2)(1 + d) with
//    d = erf(y / sqrt 2), |d| < 0.8 |y| < 2^-9.3, which is less than half the
//    distance from y / 2 to either bf16 neighbour (at least 2^-9 relative,
//    also below a power of two);
//  * |y| < 2^-125 (y = k 2^-133, k < 256): y / 2 on the 2^-133 grid; when
//    k is odd y / 2 is a tie, and as GELU(y) > y / 2 for every y != 0 it
//    rounds up: away from zero for y > 0, toward it for y < 0;
//  * |y| >= 16: y Phi(-|y|) < 16 e^-128 makes GELU(y) round to y for y > 0
//    and to -0 for y < 0 (below half of bf16's smallest subnormal);
//  * +inf -> +inf, -inf -> NaN (-inf * 0), NaN -> NaN.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gelu_table.h"

namespace svdq {

constexpr uint32_t kGeluExpLo = 118;  // exponent field of 2^-9
constexpr uint32_t kGeluExpHi = 130;  // exponent field of 8 (|y| < 16)

// The table's range holds nearly every value a layer produces: its lookup is
// the straight-line path, the other rules one branch that lanes seldom take.
__device__ __forceinline__ uint32_t gelu_bf16_bits(uint32_t b, const uint16_t *table) {
    const uint32_t sign = b & 0x8000u;
    const uint32_t e = (b >> 7) & 0xFFu;
    const uint32_t d = e - kGeluExpLo;  // wraps for e < kGeluExpLo
    const bool mid = d <= kGeluExpHi - kGeluExpLo;
    uint32_t r = table[mid ? (sign ? kGeluTableEntries / 2 : 0u) + d * 128u + (b & 0x7Fu) : 0u];
    if (__builtin_expect(!mid, 0)) {
        const uint32_t tiny = sign | (((b & 0x7FFFu) + (sign ? 0u : 1u)) >> 1);  // |y| < 2^-125
        const uint32_t half = b - 0x80u;                                          // y / 2
        const uint32_t special = b == 0x7F80u ? b : 0x7FC0u;                      // inf, NaN
        const uint32_t big = e == 0xFFu ? special : (sign ? 0x8000u : b);         // |y| >= 16
        r = e < kGeluExpLo ? (e < 2u ? tiny : half) : big;
    }
    return r;
}

}  // namespace svdq
