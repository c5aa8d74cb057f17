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

// The GEMM: C^T tile = A . B^T with A = weight rows (output columns n, K
// contiguous int8) and B = activation code rows (tokens m), on gfx950
// v_mfma_i32_32x32x32_i8 with int32 accumulation over all of K.
//  - Block 128 (n) x 128 (m), 4 waves as 2 x 2, wave tile 64 x 64 (2 x 2
//    MFMA tiles of 32 x 32).
//  - One LDS stage is 128 bytes of K (k0 .. k0 + 127) for the block's 128
//    rows of each operand: 16 KB each, double buffered (64 KB per block).
//  - Operands go straight from global memory to LDS (buffer_load ... lds,
//    16 bytes per lane, lane l to base + 16 l): 8 lanes cover one row's
//    128 bytes, so every 1 KB load reads 8 whole cache lines.
//  - In LDS the 16-byte chunk c of row r sits at chunk position
//    c ^ ((r >> 1) & 7), so the 16-byte operand reads of 16 consecutive rows
//    fall on distinct banks; a lane fetches the global chunk that belongs at
//    the position it writes.
//  - Rows past M or N and a trailing half stage (K % 128 == 64) read zeros:
//    the whole offset is in the per-lane offset, so the buffer range check
//    sees it, and chunks past K get an offset past every buffer.
constexpr int W8_TILE = 128;    // rows per block and operand
constexpr int W8_KS = 128;      // K bytes per stage
constexpr int W8_THREADS = 256;
constexpr uint32_t kW8Oob = 0x80000000u;

struct W8Stage {
    uint8_t a[W8_TILE * W8_KS];
    uint8_t b[W8_TILE * W8_KS];
};

typedef __attribute__((address_space(3))) void w8_lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w8_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

template <W8Epilogue kEpi>
__global__ __launch_bounds__(W8_THREADS, 2) void w8a8_gemm_kernel(
    const int8_t *__restrict__ qx, const int8_t *__restrict__ qw, const float *__restrict__ sxp,
    float sw, const uint16_t *__restrict__ bias, int M, int N, int K, uint16_t *__restrict__ Y,
    int32_t *__restrict__ acc_out, int tiles_n) {
    // two stages in separate LDS variables: the compiler can then tell the
    // stage being refilled (direct-to-LDS loads) from the one being read and
    // does not make the reads wait for the loads
    __shared__ __attribute__((aligned(16))) W8Stage st0;
    __shared__ __attribute__((aligned(16))) W8Stage st1;
    __shared__ __attribute__((aligned(16))) float bias_s[W8_TILE];

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int n0 = tile_n * W8_TILE;
    const int m0 = tile_m * W8_TILE;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int S = (K + W8_KS - 1) / W8_KS;

    const __amdgpu_buffer_rsrc_t ra = w8_rsrc(qw, (uint32_t)N * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t rb = w8_rsrc(qx, (uint32_t)M * (uint32_t)K);

    // Wave w issues loads 8w .. 8w + 7 of the stage's 32 (16 per operand):
    // load j of an operand fills staged rows 8 j .. 8 j + 7; lane l writes
    // row 8 j + l / 8 at chunk position l % 8.
    const int op = wave >> 1;  // waves 0, 1: weights; 2, 3: activations
    const int row0 = op ? m0 : n0;
    uint32_t gbase[8];
    int gchunk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = (wave & 1) * 8 + i;
        const int r = j * 8 + lane / 8;
        const int c = (lane % 8) ^ ((r >> 1) & 7);
        gchunk[i] = c;
        gbase[i] = (uint32_t)(row0 + r) * (uint32_t)K + (uint32_t)(c * 16);
    }
    auto issue_stage = [&](int s, W8Stage &st) {
        const int k0 = s * W8_KS;
        const bool half = k0 + W8_KS > K;  // trailing 64 bytes only
        uint8_t *dst = (op ? st.b : st.a) + (wave & 1) * 8 * 1024;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t off = gbase[i] + (uint32_t)k0;
            if (half && k0 + gchunk[i] * 16 >= K) off = kW8Oob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? rb : ra, (w8_lds_void *)(dst + i * 1024), 16, off,
                                                     0, 0, 0);
        }
    };
    // this lane's operand reads: row, and chunk position of chunk c = 2 kk + lh
    int ara[2], arb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        ara[i] = wn * 64 + i * 32 + r32;
        arb[i] = wm * 64 + i * 32 + r32;
    }
    auto frag = [&](const uint8_t *base, int r, int kk) {
        const int c = (2 * kk + lh) ^ ((r >> 1) & 7);
        return *reinterpret_cast<const i32x4 *>(base + r * W8_KS + c * 16);
    };

    i32x16 P[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) P[i][j][e] = 0;

    if constexpr (kEpi == W8Epilogue::kLinear) stage_bias_128(bias_s, bias, n0, N, threadIdx.x);
    issue_stage(0, st0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // stage s is read from `cur` while stage s + 1 loads into `nxt`
    auto run_stage = [&](int s, const W8Stage &cur, W8Stage &nxt) {
        if (s + 1 < S) issue_stage(s + 1, nxt);
#pragma unroll
        for (int kk = 0; kk < W8_KS / 32; ++kk) {
            i32x4 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = frag(cur.a, ara[i], kk);
                b[i] = frag(cur.b, arb[i], kk);
            }
#pragma unroll
            for (int in = 0; in < 2; ++in)
#pragma unroll
                for (int im = 0; im < 2; ++im) P[in][im] = mfma_i8_32x32x32(a[in], b[im], P[in][im]);
        }
        // the next stage must have landed before anyone reads it, and
        // everyone must be done with this one before it is refilled; the
        // scheduling barrier keeps this stage's MFMAs above the wait
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int s = 0; s < S; s += 2) {
        run_stage(s, st0, st1);
        if (s + 1 < S) run_stage(s + 1, st1, st0);
    }

    if constexpr (kEpi == W8Epilogue::kLinear) {
        // y = P sx sw + bias, the product rounded to fp32 before the sum
        const float scale = (*sxp) * sw;
        f32x16 acc[2][2];
#pragma unroll
        for (int in = 0; in < 2; ++in)
#pragma unroll
            for (int im = 0; im < 2; ++im)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[in][im][e] = (float)P[in][im][e] * scale;
        // every stage has been read: the stage buffers hold the output tile
        // on its way out
        static_assert(sizeof(W8Stage) >= kTileHalfLdsBytes, "LDS too small for the output tile");
        store_tile_128x128(acc, reinterpret_cast<uint8_t *>(&st0), reinterpret_cast<uint8_t *>(&st1), bias_s, Y,
                           false, M, N, m0, n0, wn, wm, threadIdx.x);
    } else {
#pragma unroll
        for (int in = 0; in < 2; ++in) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 64 + in * 32 + 8 * q + 4 * lh;
                if (n >= N) continue;
#pragma unroll
                for (int im = 0; im < 2; ++im) {
                    const int m = m0 + wm * 64 + im * 32 + r32;
                    if (m >= M) continue;
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
    const int tiles_n = (N + W8_TILE - 1) / W8_TILE;
    const int tiles_m = (M + W8_TILE - 1) / W8_TILE;
    hipLaunchKernelGGL(w8a8_gemm_kernel<W8Epilogue::kLinear>, dim3(tiles_n * tiles_m), dim3(W8_THREADS),
                       0, stream, codes, qw, scale, sw, bias, M, N, K, Y, nullptr, tiles_n);
    return hipGetLastError();
}

hipError_t launch_w8a8_acc(const int8_t *qx, const int8_t *qw, int M, int N, int K, int32_t *acc,
                           hipStream_t stream) {
    const int tiles_n = (N + W8_TILE - 1) / W8_TILE;
    const int tiles_m = (M + W8_TILE - 1) / W8_TILE;
    hipLaunchKernelGGL(w8a8_gemm_kernel<W8Epilogue::kAcc>, dim3(tiles_n * tiles_m), dim3(W8_THREADS), 0,
                       stream, qx, qw, nullptr, 0.0f, nullptr, M, N, K, nullptr, acc, tiles_n);
    return hipGetLastError();
}

}  // namespace svdq
