// The INT8 tensorwise W8A8 linear.
//
// Source: "SVDQuant ускоряет Krea 2 вдвое даже на старых NVIDIA GPU..."
// (ainews.so), section "Решение: INT8 и W4A4": INT8 "tensorwise" -- one scale
// for the whole tensor -- on the integer tensor units.
//
//   sx  = fp32(max |X| / 127)                       (dynamic, this X)
//   qx  = clamp(round-half-even(fp32(X / sx)), -127, 127)
//   acc = sum_k qx[m, k] qw[n, k]                   (int32, all of K)
//   Y   = bf16(fp32(acc) * fp32(sx * sw) + bias[n])
//
// Three launches on one stream: a grid of partial absmax values (no atomics;
// a max is order-independent, so the result is deterministic), the
// quantization pass (each block first folds the partials into sx), and the
// GEMM on gfx950 i8 MFMA.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "gemm_int.h"
#include "internal.h"

namespace svdq {

namespace {

constexpr int kPartials = 1024;
constexpr size_t kWsScaleOff = 4096;
constexpr size_t kWsCodesOff = 8192;
constexpr int kQThreads = 256;

__global__ __launch_bounds__(kQThreads) void w8_absmax_kernel(const uint16_t *__restrict__ X,
                                                              int64_t chunks,
                                                              uint32_t *__restrict__ partial) {
    uint32_t mx = 0u;
    for (int64_t c = (int64_t)blockIdx.x * kQThreads + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * kQThreads) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(X + c * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mx = max(mx, (v[i] & 0x7FFFu) << 16);
            mx = max(mx, (v[i] >> 16 & 0x7FFFu) << 16);
        }
    }
    __shared__ uint32_t red[kQThreads];
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int s = kQThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kQThreads) void w8_quantize_kernel(const uint16_t *__restrict__ X,
                                                                int64_t chunks,
                                                                const uint32_t *__restrict__ partial,
                                                                int nparts, float *__restrict__ scale_out,
                                                                int8_t *__restrict__ q) {
    __shared__ uint32_t red[kQThreads];
    uint32_t mx = 0u;
    for (int i = threadIdx.x; i < nparts; i += kQThreads) mx = max(mx, partial[i]);
    red[threadIdx.x] = mx;
    __syncthreads();
    for (int s = kQThreads / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + s]);
        __syncthreads();
    }
    const float sx = __uint_as_float(red[0]) / 127.0f;
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = sx;
    for (int64_t c = (int64_t)blockIdx.x * kQThreads + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * kQThreads) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(X + c * 8);
        uint32_t out[2] = {0u, 0u};
        if (sx != 0.0f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t h = (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu);
                float r = rintf(bf16_bits_to_f32(h) / sx);  // IEEE division, half-even
                r = fminf(127.0f, fmaxf(-127.0f, r));
                out[i >> 2] |= ((uint32_t)((int)r) & 0xFFu) << (8 * (i & 3));
            }
        }
        *reinterpret_cast<u32x2 *>(q + c * 8) = u32x2{out[0], out[1]};
    }
}

enum class W8Epilogue { kLinear, kAcc };

template <W8Epilogue kEpi>
__global__ __launch_bounds__(kGemmThreads, 2) void w8a8_gemm_kernel(
    const int8_t *__restrict__ qx, const int8_t *__restrict__ qw, const float *__restrict__ sxp,
    float sw, const uint16_t *__restrict__ bias, int M, int N, int K, uint16_t *__restrict__ Y,
    int32_t *__restrict__ acc_out, int tiles_n) {
    __shared__ GemmStage stage[2];

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
    const int S = K / kKStep;
    const uint8_t *A = reinterpret_cast<const uint8_t *>(qw);
    const uint8_t *B = reinterpret_cast<const uint8_t *>(qx);

    i32x16 P[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) P[i][j][e] = 0;

    StepRegs<false> regs;
    load_step<false, false>(regs, A, B, nullptr, nullptr, n0, m0, N, M, K, 0);
    store_step<false>(stage[0], regs);
    __syncthreads();
    for (int s = 0; s < S; ++s) {
        if (s + 1 < S) load_step<false, false>(regs, A, B, nullptr, nullptr, n0, m0, N, M, K, s + 1);
        mma_step(stage[s & 1], wn, wm, P);
        if (s + 1 < S) store_step<false>(stage[(s + 1) & 1], regs);
        __syncthreads();
    }

    float scale = 0.0f;
    if constexpr (kEpi == W8Epilogue::kLinear) scale = (*sxp) * sw;
#pragma unroll
    for (int in = 0; in < 2; ++in) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn * 64 + in * 32 + 8 * q + 4 * lh;
            if (n >= N) continue;
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if (kEpi == W8Epilogue::kLinear && bias) {
                const u32x2 bb = *reinterpret_cast<const u32x2 *>(bias + n);
                bv[0] = bf16_bits_to_f32(bb[0] & 0xFFFFu);
                bv[1] = bf16_bits_to_f32(bb[0] >> 16);
                bv[2] = bf16_bits_to_f32(bb[1] & 0xFFFFu);
                bv[3] = bf16_bits_to_f32(bb[1] >> 16);
            }
#pragma unroll
            for (int im = 0; im < 2; ++im) {
                const int m = m0 + wm * 64 + im * 32 + r32;
                if (m >= M) continue;
                if constexpr (kEpi == W8Epilogue::kLinear) {
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = (float)P[in][im][4 * q + t] * scale + bv[t];
                    const uint32_t lo = bf16x2_bits(v[0], v[1]);
                    const uint32_t hi = bf16x2_bits(v[2], v[3]);
                    *reinterpret_cast<u32x2 *>(Y + (size_t)m * N + n) = u32x2{lo, hi};
                } else {
                    i32x4 v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = P[in][im][4 * q + t];
                    *reinterpret_cast<i32x4 *>(acc_out + (size_t)m * N + n) = v;
                }
            }
        }
    }
}

}  // namespace

size_t w8a8_workspace_size(int M, int K) {
    const size_t codes = (size_t)M * (size_t)K;
    return kWsCodesOff + ((codes + 255) / 256) * 256;
}

hipError_t launch_w8a8_linear(const uint16_t *X, const int8_t *qw, float sw, const uint16_t *bias,
                              int M, int N, int K, void *workspace, uint16_t *Y,
                              hipStream_t stream) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *partial = reinterpret_cast<uint32_t *>(ws);
    float *scale = reinterpret_cast<float *>(ws + kWsScaleOff);
    int8_t *codes = reinterpret_cast<int8_t *>(ws + kWsCodesOff);
    const int64_t chunks = (int64_t)M * K / 8;
    int64_t blocks = (chunks + kQThreads * 4 - 1) / (kQThreads * 4);
    const int nparts = (int)std::max<int64_t>(1, std::min<int64_t>(kPartials, blocks));
    hipLaunchKernelGGL(w8_absmax_kernel, dim3(nparts), dim3(kQThreads), 0, stream, X, chunks, partial);
    int qblocks = (int)std::max<int64_t>(1, std::min<int64_t>(4096, (chunks + kQThreads - 1) / kQThreads));
    hipLaunchKernelGGL(w8_quantize_kernel, dim3(qblocks), dim3(kQThreads), 0, stream, X, chunks, partial,
                       nparts, scale, codes);
    const int tiles_n = (N + kTileN - 1) / kTileN;
    const int tiles_m = (M + kTileM - 1) / kTileM;
    hipLaunchKernelGGL(w8a8_gemm_kernel<W8Epilogue::kLinear>, dim3(tiles_n * tiles_m), dim3(kGemmThreads),
                       0, stream, codes, qw, scale, sw, bias, M, N, K, Y, nullptr, tiles_n);
    return hipGetLastError();
}

hipError_t launch_w8a8_acc(const int8_t *qx, const int8_t *qw, int M, int N, int K, int32_t *acc,
                           hipStream_t stream) {
    const int tiles_n = (N + kTileN - 1) / kTileN;
    const int tiles_m = (M + kTileM - 1) / kTileM;
    hipLaunchKernelGGL(w8a8_gemm_kernel<W8Epilogue::kAcc>, dim3(tiles_n * tiles_m), dim3(kGemmThreads), 0,
                       stream, qx, qw, nullptr, 0.0f, nullptr, M, N, K, nullptr, acc, tiles_n);
    return hipGetLastError();
}

}  // namespace svdq
