// The MLP pair on the device, second half: the down-projection's low-rank T
// from the per-column-tile partial sums the up-projection's MLP epilogue
// wrote; and the same GELU rule as an elementwise pass (the entry point that
// checks the device's GELU on every bf16 input, and the unfused pipeline's
// GELU step in the benchmark).
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
// paragraph (the 16-bit low-rank branch: T = X L1s rounded once to bf16) and
// "Nunchaku Lite" paragraph (svdq_w4a4 on the MLP projections, fused kernels).

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "gelu.h"
#include "internal.h"

namespace svdq {

namespace {

// T[m, j] = bf16(sum over column tiles c, in ascending order, of
// tpart[c, m, j]): deterministic. Each thread sums four consecutive elements
// (16-byte loads of the partials, one 8-byte store of T; n = M * rank is a
// multiple of 16 and the workspace 16-byte aligned), or one where T is not
// 8-byte aligned.
template <int kVec>
__global__ __launch_bounds__(256) void tpart_reduce_kernel(const float *__restrict__ tpart, int parts, int M,
                                                           int rank, uint16_t *__restrict__ T) {
    typedef float fv __attribute__((ext_vector_type(kVec)));
    const size_t n = (size_t)M * rank;
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * kVec;
    if (i >= n) return;
    // loads eight partials ahead of the adds (the adds stay in order)
    fv v = {};
    int c = 0;
    for (; c + 8 <= parts; c += 8) {
        fv p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = *reinterpret_cast<const fv *>(tpart + (size_t)(c + j) * n + i);
#pragma unroll
        for (int j = 0; j < 8; ++j) v += p[j];
    }
    for (; c < parts; ++c) v += *reinterpret_cast<const fv *>(tpart + (size_t)c * n + i);
    if constexpr (kVec == 4) {
        *reinterpret_cast<u32x2 *>(T + i) = u32x2{f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                                                  f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16)};
    } else {
        T[i] = (uint16_t)f32_to_bf16_bits(v[0]);
    }
}

// Elementwise GELU: each block loads the table into LDS once and handles
// kGeluPerBlock elements; with 16-byte aligned pointers as 8-value vectors
// (32 values per thread), else one value at a time.
constexpr int kGeluPerBlock = 256 * 32;

__global__ __launch_bounds__(256) void gelu_bf16_kernel(const uint16_t *__restrict__ y, uint16_t *__restrict__ g,
                                                        int n, bool vec) {
    __shared__ __attribute__((aligned(16))) uint16_t tab[kGeluTableEntries];
    for (int i = threadIdx.x; i < kGeluTableEntries / 8; i += 256)
        reinterpret_cast<u32x4 *>(tab)[i] = reinterpret_cast<const u32x4 *>(kGeluTable)[i];
    __syncthreads();
    const int base = blockIdx.x * kGeluPerBlock;
    if (vec) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int e = base + 8 * (k * 256 + (int)threadIdx.x);
            if (e + 8 <= n) {
                u32x4 w = *reinterpret_cast<const u32x4 *>(y + e);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[j] = gelu_bf16_bits(w[j] & 0xFFFFu, tab) | (gelu_bf16_bits(w[j] >> 16, tab) << 16);
                *reinterpret_cast<u32x4 *>(g + e) = w;
            } else {
                for (int i = e; i < min(e + 8, n); ++i) g[i] = (uint16_t)gelu_bf16_bits(y[i], tab);
            }
        }
    } else {
        for (int i = base + (int)threadIdx.x; i < min(base + kGeluPerBlock, n); i += 256)
            g[i] = (uint16_t)gelu_bf16_bits(y[i], tab);
    }
}

}  // namespace

hipError_t launch_tpart_reduce(const float *tpart, int parts, int M, int rank, uint16_t *T, hipStream_t stream) {
    const size_t n = (size_t)M * rank;
    if (n == 0) return hipSuccess;
    if ((n % 4) == 0 && (reinterpret_cast<uintptr_t>(T) & 7u) == 0 && (reinterpret_cast<uintptr_t>(tpart) & 15u) == 0) {
        const size_t threads = n / 4;
        hipLaunchKernelGGL(tpart_reduce_kernel<4>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                           tpart, parts, M, rank, T);
    } else {
        hipLaunchKernelGGL(tpart_reduce_kernel<1>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, tpart,
                           parts, M, rank, T);
    }
    return hipGetLastError();
}

hipError_t launch_gelu_bf16(const uint16_t *y, uint16_t *g, int n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const bool vec = (((uintptr_t)y | (uintptr_t)g) & 15u) == 0;
    hipLaunchKernelGGL(gelu_bf16_kernel, dim3((unsigned)((n + kGeluPerBlock - 1) / kGeluPerBlock)), dim3(256), 0,
                       stream, y, g, n, vec);
    return hipGetLastError();
}

}  // namespace svdq
