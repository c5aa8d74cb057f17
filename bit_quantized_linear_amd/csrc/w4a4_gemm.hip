// The SVDQuant W4A4 linear: INT4 x INT4 GEMM with per-group scaling, fused
// with the 16-bit low-rank up-projection and the bias.
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
// paragraph (4-bit weights x 4-bit activations with a 16-bit low-rank branch)
// and "Nunchaku Lite" paragraph (svdq_w4a4 layers for the attention and MLP
// projections, INT4 variant). Grouped INT4 format: "Diffusion Compiler"
// README, "Compiler" bullet.
//
//   P[g, m, n] = sum_{k in g} qx[m, k] qw[n, k]          (int32, exact)
//   acc[m, n] += fp32(sx[g, m] sw[g, n]) * P[g, m, n]     (fp32, g ascending)
//   y = acc + T L2 + bias  ->  bf16 (nearest even) or fp32
//
// The nibbles are unpacked to 16 * code, so the MFMA sums 256 * P. The main
// loop accumulates acc' = sum_g fp32(sx sw) (256 P) -- 256 times the fp32
// accumulator of the formula above at every step, since a power-of-two factor
// commutes with each rounding -- and acc = acc' / 256 is taken once before the
// low-rank branch is added. The scale product is rounded where the formula
// rounds it, also for groups so small that it is a subnormal fp32 (folding
// 1/256 into the scale instead would push such products 8 binades further
// into the subnormal range and lose their precision).

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "gemm_int.h"
#include "internal.h"

namespace svdq {

namespace {

enum class W4Epilogue { kLinear, kPartials };

template <W4Epilogue kEpi>
__global__ __launch_bounds__(kGemmThreads, 2) void w4a4_gemm_kernel(
    const uint8_t *__restrict__ qx, const float *__restrict__ sx, const uint16_t *__restrict__ T,
    const uint8_t *__restrict__ qw, const float *__restrict__ sw, const uint16_t *__restrict__ l2t,
    const uint16_t *__restrict__ bias, int M, int N, int K, int rank, void *__restrict__ Y,
    bool y_f32, int32_t *__restrict__ Pout, int tiles_n) {
    __shared__ __attribute__((aligned(16))) GemmStage stage[2];
    __shared__ __attribute__((aligned(16))) float bias_s[kTileN];

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int n0 = tile_n * kTileN;
    const int m0 = tile_m * kTileM;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int G = K / kKStep;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    StepRegs<true> regs;
    load_step<true, kEpi == W4Epilogue::kLinear>(regs, qw, qx, sw, sx, n0, m0, N, M, K, 0);
    store_step<true>(stage[0], regs);
    if constexpr (kEpi == W4Epilogue::kLinear) stage_bias_128(bias_s, bias, n0, N, threadIdx.x);
    __syncthreads();

    for (int g = 0; g < G; ++g) {
        const GemmStage &cur = stage[g & 1];
        if (g + 1 < G) load_step<true, kEpi == W4Epilogue::kLinear>(regs, qw, qx, sw, sx, n0, m0, N, M, K, g + 1);

        i32x16 P[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) P[i][j][e] = 0;
        mma_step(cur, wn, wm, P);

        if constexpr (kEpi == W4Epilogue::kLinear) {
            // rows of the 32x32 output are weight rows n = 8q + 4 lh + t,
            // the column is the token m = r32
            float sxm[2];
#pragma unroll
            for (int im = 0; im < 2; ++im) sxm[im] = cur.sb[wm * 64 + im * 32 + r32];
#pragma unroll
            for (int in = 0; in < 2; ++in) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 s4 = *reinterpret_cast<const f32x4 *>(&cur.sa[wn * 64 + in * 32 + 8 * q + 4 * lh]);
#pragma unroll
                    for (int im = 0; im < 2; ++im) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const float scale = sxm[im] * s4[t];
                            acc[in][im][4 * q + t] = fmaf(scale, (float)P[in][im][4 * q + t], acc[in][im][4 * q + t]);
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int in = 0; in < 2; ++in) {
#pragma unroll
                for (int im = 0; im < 2; ++im) {
                    const int m = m0 + wm * 64 + im * 32 + r32;
                    if (m >= M) continue;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = n0 + wn * 64 + in * 32 + 8 * q + 4 * lh;
                        if (n >= N) continue;
                        i32x4 v;
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = P[in][im][4 * q + t] >> 8;
                        *reinterpret_cast<i32x4 *>(Pout + ((size_t)g * M + m) * N + n) = v;
                    }
                }
            }
        }

        if (g + 1 < G) store_step<true>(stage[(g + 1) & 1], regs);
        __syncthreads();
    }

    if constexpr (kEpi == W4Epilogue::kLinear) {
        // acc = acc' / 256 (exact while acc is a normal fp32 number; a result
        // in the subnormal range is rounded once more, by at most half of
        // 2^-149)
#pragma unroll
        for (int in = 0; in < 2; ++in)
#pragma unroll
            for (int im = 0; im < 2; ++im)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[in][im][e] *= 1.0f / 256.0f;
        // low-rank up-projection: C^T += L2^T-rows (A, weight side) x T-rows
        // (B, token side) on bf16 MFMA, K = rank in slices of 16
        for (int kk = 0; kk < rank; kk += 16) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int n = n0 + wn * 64 + i * 32 + r32;
                const int m = m0 + wm * 64 + i * 32 + r32;
                u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
                if (n < N) va = *reinterpret_cast<const u32x4 *>(l2t + (size_t)n * rank + kk + 8 * lh);
                if (m < M) vb = *reinterpret_cast<const u32x4 *>(T + (size_t)m * rank + kk + 8 * lh);
                a[i] = __builtin_bit_cast(bf16x8, va);
                b[i] = __builtin_bit_cast(bf16x8, vb);
            }
#pragma unroll
            for (int in = 0; in < 2; ++in)
#pragma unroll
                for (int im = 0; im < 2; ++im) acc[in][im] = mfma_bf16_32x32x16(a[in], b[im], acc[in][im]);
        }
        // every stage has been read: the stage buffers hold the output tile on
        // its way out
        static_assert(sizeof(GemmStage) >= kTileHalfLdsBytes, "LDS too small for the output tile");
        store_tile_128x128(acc, reinterpret_cast<uint8_t *>(&stage[0]), reinterpret_cast<uint8_t *>(&stage[1]),
                           bias_s, Y, y_f32, M, N, m0, n0, wn, wm, threadIdx.x);
    }
}

}  // namespace

hipError_t launch_w4a4_linear(const uint8_t *qx, const float *sx, const uint16_t *T,
                              const uint8_t *qw, const float *sw, const uint16_t *l2t,
                              const uint16_t *bias, int M, int N, int K, int rank, void *Y,
                              bool y_f32, hipStream_t stream) {
    const int tiles_n = (N + kTileN - 1) / kTileN;
    const int tiles_m = (M + kTileM - 1) / kTileM;
    hipLaunchKernelGGL(w4a4_gemm_kernel<W4Epilogue::kLinear>, dim3(tiles_n * tiles_m),
                       dim3(kGemmThreads), 0, stream, qx, sx, T, qw, sw, l2t, bias, M, N, K, rank,
                       Y, y_f32, nullptr, tiles_n);
    return hipGetLastError();
}

hipError_t launch_w4a4_partials(const uint8_t *qx, const uint8_t *qw, int M, int N, int K,
                                int32_t *P, hipStream_t stream) {
    const int tiles_n = (N + kTileN - 1) / kTileN;
    const int tiles_m = (M + kTileM - 1) / kTileM;
    hipLaunchKernelGGL(w4a4_gemm_kernel<W4Epilogue::kPartials>, dim3(tiles_n * tiles_m),
                       dim3(kGemmThreads), 0, stream, qx, nullptr, nullptr, qw, nullptr, nullptr,
                       nullptr, M, N, K, 0, nullptr, false, P, tiles_n);
    return hipGetLastError();
}

}  // namespace svdq
