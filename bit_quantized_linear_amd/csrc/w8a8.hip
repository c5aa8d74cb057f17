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
#include "quant_common.h"

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
    // x / sx as fp32(double(x) * fp64(1 / sx)): the same value as the IEEE
    // fp32 division (quotient_fp32). A quotient below 2^-126, where that
    // argument does not hold, is code 0 either way.
    const double rsx = sx != 0.0f ? 1.0 / (double)sx : 0.0;
    for (int64_t c = (int64_t)blockIdx.x * kQThreads + threadIdx.x; c < chunks;
         c += (int64_t)gridDim.x * kQThreads) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(X + c * 8);
        uint32_t out[2] = {0u, 0u};
        if (sx != 0.0f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t h = (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu);
                float r = rintf(quotient_fp32(bf16_bits_to_f32(h), rsx));  // half-even
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
//  - Block 256 (n) x 256 (m), 8 waves as 2 x 4, wave tile 128 x 64 (4 x 2
//    MFMA tiles of 32 x 32).
//  - One LDS stage is 128 bytes of K (k0 .. k0 + 127) for the block's 256
//    rows of each operand: 32 KB each, double buffered (128 KB per block,
//    one block of 8 waves per CU); a stage is 32 MFMAs per wave, long
//    enough for the next stage's loads to land.
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
//  - Against a 128 x 128 tile with the same staging (4 waves, two blocks
//    per CU): 10-13 % faster at 32760 x 5120 x 5120, 5 % at 4608 x 3072 x
//    3072, half the operand bytes per multiply-add.
//  - Fragment reads run one 32-byte step ahead of the MFMAs, also across
//    the stage barrier: 4-5 % faster at 32760 x 5120 x 5120, 5-10 % at
//    4608 x 3072 x 3072 and 13 % at 1000 x 3072 x 3072 than reading each
//    step's fragments right before its MFMAs.
constexpr uint32_t kW8Oob = 0x80000000u;

typedef __attribute__((address_space(3))) void w8_lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w8_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

constexpr int WB_TILE = 256;
constexpr int WB_KS = 128;
constexpr int WB_THREADS = 512;
constexpr int WB_PITCH = 2 * WB_TILE + 16;  // bytes per output row staged in LDS (bf16, padded)

struct WbStage {
    uint8_t a[WB_TILE * WB_KS];
    uint8_t b[WB_TILE * WB_KS];
};

template <W8Epilogue kEpi>
__global__ __launch_bounds__(WB_THREADS, 1) void w8a8_gemm256_kernel(
    const int8_t *__restrict__ qx, const int8_t *__restrict__ qw, const float *__restrict__ sxp,
    float sw, const uint16_t *__restrict__ bias, int M, int N, int K, uint16_t *__restrict__ Y,
    int32_t *__restrict__ acc_out, int tiles_n) {
    __shared__ __attribute__((aligned(16))) WbStage st0;
    __shared__ __attribute__((aligned(16))) WbStage st1;
    __shared__ __attribute__((aligned(16))) float bias_s[WB_TILE];

    // blocks are dealt to the 8 XCDs round-robin (block b runs on XCD
    // b % 8): XCD c takes the contiguous tile range [c T / 8, (c + 1) T / 8),
    // walked four m-tiles at a time across n, so that the tiles an XCD runs
    // together share operand rows in its L2
    int tile_n, tile_m;
    {
        const int T = gridDim.x;
        const int b = blockIdx.x;
        const int id = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
        const int tiles_m = T / tiles_n;
        const int group = id / (4 * tiles_n);
        const int first_m = group * 4;
        const int gm = min(4, tiles_m - first_m);
        const int in_group = id - group * 4 * tiles_n;
        tile_m = first_m + in_group % gm;
        tile_n = in_group / gm;
    }
    const int n0 = tile_n * WB_TILE;
    const int m0 = tile_m * WB_TILE;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int S = (K + WB_KS - 1) / WB_KS;

    const __amdgpu_buffer_rsrc_t ra = w8_rsrc(qw, (uint32_t)N * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t rb = w8_rsrc(qx, (uint32_t)M * (uint32_t)K);

    // waves 0-3 issue the weights' 32 loads of a stage, waves 4-7 the
    // activations'; load j fills staged rows 8 j .. 8 j + 7, lane l row
    // 8 j + l / 8 at chunk position l % 8
    const int op = wave >> 2;
    const int row0 = op ? m0 : n0;
    uint32_t gbase[8];
    int gchunk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = (wave & 3) * 8 + i;
        const int r = j * 8 + lane / 8;
        const int c = (lane % 8) ^ ((r >> 1) & 7);
        gchunk[i] = c;
        gbase[i] = (uint32_t)(row0 + r) * (uint32_t)K + (uint32_t)(c * 16);
    }
    auto issue_stage = [&](int s, WbStage &st) __attribute__((always_inline)) {
        const int k0 = s * WB_KS;
        const bool half = k0 + WB_KS > K;  // trailing 64 bytes only
        uint8_t *dst = (op ? st.b : st.a) + (wave & 3) * 8 * 1024;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t off = gbase[i] + (uint32_t)k0;
            if (half && k0 + gchunk[i] * 16 >= K) off = kW8Oob;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op ? rb : ra, (w8_lds_void *)(dst + i * 1024), 16, off,
                                                     0, 0, 0);
        }
    };
    auto frag = [&](const uint8_t *base, int r, int kk) __attribute__((always_inline)) {
        const int c = (2 * kk + lh) ^ ((r >> 1) & 7);
        return *reinterpret_cast<const i32x4 *>(base + r * WB_KS + c * 16);
    };

    i32x16 P[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) P[i][j][e] = 0;

    if constexpr (kEpi == W8Epilogue::kLinear)
        if (tid < WB_TILE) bias_s[tid] = bias && n0 + tid < N ? bf16_bits_to_f32(bias[n0 + tid]) : 0.0f;
    issue_stage(0, st0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // The fragments of step kk + 1 are read while the MFMAs of step kk run
    // (two fragment sets), and the stage barrier sits before the last
    // step's MFMAs, so that the next stage's first fragments are read while
    // they run: no LDS read latency is waited for in front of an MFMA group.
    i32x4 fa[2][4], fb[2][2];
    auto read_step = [&](const WbStage &cur, int kk, i32x4 (&a)[4], i32x4 (&b)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = frag(cur.a, wn * 128 + i * 32 + r32, kk);
#pragma unroll
        for (int i = 0; i < 2; ++i) b[i] = frag(cur.b, wm * 64 + i * 32 + r32, kk);
    };
    auto mfma_step = [&](const i32x4 (&a)[4], const i32x4 (&b)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int in = 0; in < 4; ++in)
#pragma unroll
            for (int im = 0; im < 2; ++im) P[in][im] = mfma_i8_32x32x32(a[in], b[im], P[in][im]);
    };
    read_step(st0, 0, fa[0], fb[0]);
    // on entry the fragments of step 0 of stage s are in set 0; steps 1-3
    // alternate sets 1, 0, 1
    auto run_stage = [&](int s, const WbStage &cur, WbStage &nxt) __attribute__((always_inline)) {
        if (s + 1 < S) issue_stage(s + 1, nxt);
#pragma unroll
        for (int kk = 0; kk < WB_KS / 32 - 1; ++kk) {
            read_step(cur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mfma_step(fa[kk & 1], fb[kk & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // every wave has read all of stage s (its last step is in set 1);
        // once the next stage has landed everywhere, its first step is read
        // while the last MFMAs of this one run
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (s + 1 < S) read_step(nxt, 0, fa[0], fb[0]);
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(fa[1], fb[1]);
        __builtin_amdgcn_sched_barrier(0);
    };
    int s = 0;
    for (; s + 1 < S; s += 2) {
        run_stage(s, st0, st1);
        run_stage(s + 1, st1, st0);
    }
    if (s < S) run_stage(s, st0, st1);
    __syncthreads();

    if constexpr (kEpi == W8Epilogue::kLinear) {
        // y = P sx sw + bias, rounded once to bf16; staged through LDS a
        // quarter (64 tokens: the waves of one wm) at a time, alternating
        // between the two stage buffers, each quarter stored as whole
        // 512-byte row segments
        const float scale = (*sxp) * sw;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint8_t *buf = reinterpret_cast<uint8_t *>((q & 1) ? &st1 : &st0);
            if (wm == q) {
#pragma unroll
                for (int in = 0; in < 4; ++in) {
#pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int nl = wn * 128 + in * 32 + 8 * qq + 4 * lh;
                        const f32x4 bv = *reinterpret_cast<const f32x4 *>(bias_s + nl);
#pragma unroll
                        for (int im = 0; im < 2; ++im) {
                            const int ml = im * 32 + r32;
                            float v[4];
#pragma unroll
                            for (int t = 0; t < 4; ++t) v[t] = (float)P[in][im][4 * qq + t] * scale + bv[t];
                            *reinterpret_cast<u32x2 *>(buf + ml * WB_PITCH + nl * 2) =
                                u32x2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
                        }
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + WB_THREADS * i;  // 64 rows x 32 pieces
                const int row = c >> 5, piece = c & 31;
                const int m = m0 + 64 * q + row, n = n0 + piece * 8;
                if (m < M && n < N)
                    *reinterpret_cast<u32x4 *>(Y + (size_t)m * N + n) =
                        *reinterpret_cast<const u32x4 *>(buf + row * WB_PITCH + piece * 16);
            }
        }
    } else {
#pragma unroll
        for (int in = 0; in < 4; ++in) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * 128 + in * 32 + 8 * q + 4 * lh;
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
    const int tiles_n = (N + WB_TILE - 1) / WB_TILE;
    const int tiles_m = (M + WB_TILE - 1) / WB_TILE;
    hipLaunchKernelGGL(w8a8_gemm256_kernel<W8Epilogue::kLinear>, dim3(tiles_n * tiles_m), dim3(WB_THREADS),
                       0, stream, codes, qw, scale, sw, bias, M, N, K, Y, nullptr, tiles_n);
    return hipGetLastError();
}

hipError_t launch_w8a8_acc(const int8_t *qx, const int8_t *qw, int M, int N, int K, int32_t *acc,
                           hipStream_t stream) {
    const int tiles_n = (N + WB_TILE - 1) / WB_TILE;
    const int tiles_m = (M + WB_TILE - 1) / WB_TILE;
    hipLaunchKernelGGL(w8a8_gemm256_kernel<W8Epilogue::kAcc>, dim3(tiles_n * tiles_m), dim3(WB_THREADS), 0,
                       stream, qx, qw, nullptr, 0.0f, nullptr, M, N, K, nullptr, acc, tiles_n);
    return hipGetLastError();
}

}  // namespace svdq
