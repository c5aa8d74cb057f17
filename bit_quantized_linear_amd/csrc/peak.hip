// Matrix-core rate measured on the device itself: back-to-back MFMAs of one
// kind on every SIMD, so that roofline fractions can be quoted against the
// rate this chip reaches under load as well as against the published peak,
// and the shader clock under that load (clock64 cycles against the 100 MHz
// real-time counter).

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace svdq {

namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kRateThreads = 256;  // 4 waves per block
constexpr int kChains = 4;         // independent accumulator chains per wave

// Each wave runs `iters` rounds of kChains independent MFMAs (enough to keep
// the matrix pipe of its SIMD busy) and writes its shader-clock and real-time
// spans to out[2 w], out[2 w + 1]. The operands are FP6 / int8 / bf16 values
// of the codes' magnitude; the results are folded into a store that never
// happens, so the MFMAs cannot be dropped.
template <int kKind>
__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(int iters, uint64_t *__restrict__ out,
                                                                 int never) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (kRateThreads / 64) + (threadIdx.x >> 6);
    f32x16 accf[kChains];
    i32x16 acci[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            accf[c][e] = 0.0f;
            acci[c][e] = 0;
        }
    }
    // FP6 E2M3 fields of codes 1..7 (value code / 8), 32 per lane half
    i32x8 a6, b6;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a6[i] = (int)(0x14514514u + (uint32_t)(lane + i));
        b6[i] = (int)(0x0C30C30Cu + (uint32_t)(lane * 3 + i));
    }
    i32x4 a8, b8;
    bf16x8 ab, bb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a8[i] = 0x05030107 + lane;
        b8[i] = 0x07010305 - lane;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ab[i] = (__bf16)(0.125f * (float)((lane + i) % 7));
        bb[i] = (__bf16)(0.25f * (float)((lane * 3 + i) % 5));
    }
    asm volatile("" : "+v"(a6), "+v"(b6), "+v"(a8), "+v"(b8));
    const uint64_t c0 = __builtin_readcyclecounter();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (kKind == 0)
                accf[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a6, b6, accf[c], 2, 2, 0, 130, 0, 130);
            else if constexpr (kKind == 1)
                acci[c] = mfma_i8_32x32x32(a8, b8, acci[c]);
            else
                accf[c] = mfma_bf16_32x32x16(ab, bb, accf[c]);
        }
    }
    const uint64_t c1 = __builtin_readcyclecounter();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
        out[2 * gw] = c1 - c0;
        out[2 * gw + 1] = r1 - r0;
    }
    float sink = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) sink += accf[c][e] + (float)acci[c][e];
    if (never == 1 && sink == 1.2345f) out[0] = 0;
}

}  // namespace

int64_t mfma_rate_ops_per_wave_round(int kind) {
    // 2 M N K per MFMA, kChains MFMAs per round
    const int64_t k = kind == 0 ? 64 : (kind == 1 ? 32 : 16);
    return 2LL * 32 * 32 * k * kChains;
}

hipError_t launch_mfma_rate(int kind, int blocks, int iters, uint64_t *out, hipStream_t stream) {
    if (kind == 0)
        hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(blocks), dim3(kRateThreads), 0, stream, iters, out, 0);
    else if (kind == 1)
        hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(blocks), dim3(kRateThreads), 0, stream, iters, out, 0);
    else
        hipLaunchKernelGGL(mfma_rate_kernel<2>, dim3(blocks), dim3(kRateThreads), 0, stream, iters, out, 0);
    return hipGetLastError();
}

}  // namespace svdq
