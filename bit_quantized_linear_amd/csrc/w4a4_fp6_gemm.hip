// The SVDQuant W4A4 linear on the FP6 container: INT4 x INT4 group products
// on gfx950's FP6 MFMA, per-group scaling, fused low-rank up-projection and
// bias.
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
// paragraph (4-bit weights x 4-bit activations with a 16-bit low-rank branch)
// and "Nunchaku Lite" paragraph (svdq_w4a4 layers for the attention and MLP
// projections).
//
//   P[g, m, n] = sum_{k in g} qx[m, k] qw[n, k]          (exact, fp32)
//   acc[m, n] += fp32(sx[g, m] sw[g, n]) * P[g, m, n]     (fp32, g ascending)
//   y = acc + T L2 + bias  ->  bf16 (nearest even) or fp32
//
// The codes -7..7 are stored as FP6 E2M3 numbers code/8; the MFMA's E8M0
// block scales (2^3 on each operand) bring the product back to integers, so
// one v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 = one group) returns the
// group's partial P exactly in fp32 (|P| <= 3136). There is no nibble unpack
// and no integer-to-float conversion; the vector ALU does one multiply (the
// scale product) and one FMA per output element and group.
//
// Block tile 256 (n) x 128 (m), 8 waves as 4 (n) x 2 (m), wave tile 64 x 64
// (2 x 2 MFMA tiles of 32 x 32). Per group a block stages 256 x 48 + 128 x 48
// bytes of codes (128-bit loads, rows padded to 56 bytes in LDS so that 32
// lanes reading 8 bytes each from 32 rows hit distinct banks) and 384
// scales; LDS is double buffered with one barrier per group and the next
// group's loads in flight during the MFMAs.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace svdq {

namespace {

constexpr int BN = 256;
constexpr int BM = 128;
constexpr int THREADS = 512;
constexpr int WAVES_N = 4;
constexpr int WTN = 64;
constexpr int WTM = 64;
constexpr int ROW6 = 56;  // LDS stride of one staged row (48 code bytes + 8 pad)
constexpr int CHUNKS_A = BN * 3;  // 16-byte chunks per group
constexpr int CHUNKS = (BN + BM) * 3;
constexpr int E8M0_X8 = 127 + 3;  // block scale 2^3

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

struct Stage6 {
    uint8_t a[BN * ROW6];
    uint8_t b[BM * ROW6];
    float sa[BN];
    float sb[BM];
};

struct Regs6 {
    u32x4 c[3];
    float s;
};

template <bool kLinear>
__device__ __forceinline__ void load6(Regs6 &r, const uint8_t *__restrict__ qw, const uint8_t *__restrict__ qx,
                                      const float *__restrict__ sw, const float *__restrict__ sx, int n0, int m0,
                                      int N, int M, size_t R, int g) {
    const int tid = threadIdx.x;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int c = tid + i * THREADS;
        r.c[i] = zero;
        if (c < CHUNKS_A) {
            const int row = c / 3, part = c - 3 * (c / 3);
            if (n0 + row < N)
                r.c[i] = *reinterpret_cast<const u32x4 *>(qw + (size_t)(n0 + row) * R + (size_t)g * 48 + part * 16);
        } else if (c < CHUNKS) {
            const int cc = c - CHUNKS_A;
            const int row = cc / 3, part = cc - 3 * (cc / 3);
            if (m0 + row < M)
                r.c[i] = *reinterpret_cast<const u32x4 *>(qx + (size_t)(m0 + row) * R + (size_t)g * 48 + part * 16);
        }
    }
    r.s = 0.0f;
    if constexpr (kLinear) {
        if (tid < BM) {
            if (m0 + tid < M) r.s = sx[(size_t)g * M + m0 + tid];
        } else if (tid < BM + BN) {
            const int j = tid - BM;
            if (n0 + j < N) r.s = sw[(size_t)g * N + n0 + j];
        }
    }
}

template <bool kLinear>
__device__ __forceinline__ void store6(Stage6 &st, const Regs6 &r) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int c = tid + i * THREADS;
        uint8_t *dst = nullptr;
        if (c < CHUNKS_A) {
            const int row = c / 3, part = c - 3 * (c / 3);
            dst = st.a + row * ROW6 + part * 16;
        } else if (c < CHUNKS) {
            const int cc = c - CHUNKS_A;
            const int row = cc / 3, part = cc - 3 * (cc / 3);
            dst = st.b + row * ROW6 + part * 16;
        }
        if (dst) {
            *reinterpret_cast<u32x2 *>(dst) = u32x2{r.c[i][0], r.c[i][1]};
            *reinterpret_cast<u32x2 *>(dst + 8) = u32x2{r.c[i][2], r.c[i][3]};
        }
    }
    if constexpr (kLinear) {
        if (tid < BM)
            st.sb[tid] = r.s;
        else if (tid < BM + BN)
            st.sa[tid - BM] = r.s;
    }
}

// 24 bytes (32 codes: lane half lh of the group) of one staged row
__device__ __forceinline__ i32x8 frag6(const uint8_t *row_base, int lh) {
    const uint8_t *p = row_base + 24 * lh;
    const u32x2 x0 = *reinterpret_cast<const u32x2 *>(p);
    const u32x2 x1 = *reinterpret_cast<const u32x2 *>(p + 8);
    const u32x2 x2 = *reinterpret_cast<const u32x2 *>(p + 16);
    return i32x8{(int)x0[0], (int)x0[1], (int)x1[0], (int)x1[1], (int)x2[0], (int)x2[1], 0, 0};
}

template <bool kLinear>
__global__ __launch_bounds__(THREADS, 1) void w4a4_fp6_kernel(
    const uint8_t *__restrict__ qx, const float *__restrict__ sx, const uint16_t *__restrict__ T,
    const uint8_t *__restrict__ qw, const float *__restrict__ sw, const uint16_t *__restrict__ l2t,
    const uint16_t *__restrict__ bias, int M, int N, int K, int rank, void *__restrict__ Y, bool y_f32,
    int32_t *__restrict__ Pout, int tiles_n) {
    __shared__ Stage6 stage[2];

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int n0 = tile_n * BN;
    const int m0 = tile_m * BM;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % WAVES_N;
    const int wm = wave / WAVES_N;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int G = K / 64;
    const size_t R = (size_t)K / 4 * 3;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    Regs6 regs;
    load6<kLinear>(regs, qw, qx, sw, sx, n0, m0, N, M, R, 0);
    store6<kLinear>(stage[0], regs);
    __syncthreads();

    for (int g = 0; g < G; ++g) {
        const Stage6 &cur = stage[g & 1];
        if (g + 1 < G) load6<kLinear>(regs, qw, qx, sw, sx, n0, m0, N, M, R, g + 1);

        i32x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a[i] = frag6(cur.a + (wn * WTN + i * 32 + r32) * ROW6, lh);
            b[i] = frag6(cur.b + (wm * WTM + i * 32 + r32) * ROW6, lh);
        }
#pragma unroll
        for (int in = 0; in < 2; ++in) {
#pragma unroll
            for (int im = 0; im < 2; ++im) {
                const f32x16 P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[in], b[im], zero16, 2, 2, 0, E8M0_X8, 0, E8M0_X8);
                if constexpr (kLinear) {
                    const float sxm = cur.sb[wm * WTM + im * 32 + r32];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4 s4 = *reinterpret_cast<const f32x4 *>(&cur.sa[wn * WTN + in * 32 + 8 * q + 4 * lh]);
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            acc[in][im][4 * q + t] = fmaf(sxm * s4[t], P[4 * q + t], acc[in][im][4 * q + t]);
                    }
                } else {
                    const int m = m0 + wm * WTM + im * 32 + r32;
                    if (m < M) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int n = n0 + wn * WTN + in * 32 + 8 * q + 4 * lh;
                            if (n < N) {
                                i32x4 v;
#pragma unroll
                                for (int t = 0; t < 4; ++t) v[t] = (int)P[4 * q + t];
                                *reinterpret_cast<i32x4 *>(Pout + ((size_t)g * M + m) * N + n) = v;
                            }
                        }
                    }
                }
            }
        }

        if (g + 1 < G) store6<kLinear>(stage[(g + 1) & 1], regs);
        __syncthreads();
    }

    if constexpr (kLinear) {
        for (int kk = 0; kk < rank; kk += 16) {
            bf16x8 la[2], lb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int n = n0 + wn * WTN + i * 32 + r32;
                const int m = m0 + wm * WTM + i * 32 + r32;
                u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
                if (n < N) va = *reinterpret_cast<const u32x4 *>(l2t + (size_t)n * rank + kk + 8 * lh);
                if (m < M) vb = *reinterpret_cast<const u32x4 *>(T + (size_t)m * rank + kk + 8 * lh);
                la[i] = __builtin_bit_cast(bf16x8, va);
                lb[i] = __builtin_bit_cast(bf16x8, vb);
            }
#pragma unroll
            for (int in = 0; in < 2; ++in)
#pragma unroll
                for (int im = 0; im < 2; ++im) acc[in][im] = mfma_bf16_32x32x16(la[in], lb[im], acc[in][im]);
        }
#pragma unroll
        for (int in = 0; in < 2; ++in) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + wn * WTN + in * 32 + 8 * q + 4 * lh;
                if (n >= N) continue;
                float bv[4] = {0.f, 0.f, 0.f, 0.f};
                if (bias) {
                    const u32x2 bb = *reinterpret_cast<const u32x2 *>(bias + n);
                    bv[0] = bf16_bits_to_f32(bb[0] & 0xFFFFu);
                    bv[1] = bf16_bits_to_f32(bb[0] >> 16);
                    bv[2] = bf16_bits_to_f32(bb[1] & 0xFFFFu);
                    bv[3] = bf16_bits_to_f32(bb[1] >> 16);
                }
#pragma unroll
                for (int im = 0; im < 2; ++im) {
                    const int m = m0 + wm * WTM + im * 32 + r32;
                    if (m >= M) continue;
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = acc[in][im][4 * q + t] + bv[t];
                    if (y_f32) {
                        *reinterpret_cast<f32x4 *>(static_cast<float *>(Y) + (size_t)m * N + n) =
                            f32x4{v[0], v[1], v[2], v[3]};
                    } else {
                        const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(Y) + (size_t)m * N + n) = u32x2{lo, hi};
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_w4a4_fp6_linear(const uint8_t *qx, const float *sx, const uint16_t *T, const uint8_t *qw,
                                  const float *sw, const uint16_t *l2t, const uint16_t *bias, int M, int N,
                                  int K, int rank, void *Y, bool y_f32, hipStream_t stream) {
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles_m = (M + BM - 1) / BM;
    hipLaunchKernelGGL(w4a4_fp6_kernel<true>, dim3(tiles_n * tiles_m), dim3(THREADS), 0, stream, qx, sx, T, qw,
                       sw, l2t, bias, M, N, K, rank, Y, y_f32, nullptr, tiles_n);
    return hipGetLastError();
}

hipError_t launch_w4a4_fp6_partials(const uint8_t *qx, const uint8_t *qw, int M, int N, int K, int32_t *P,
                                    hipStream_t stream) {
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles_m = (M + BM - 1) / BM;
    hipLaunchKernelGGL(w4a4_fp6_kernel<false>, dim3(tiles_n * tiles_m), dim3(THREADS), 0, stream, qx, nullptr,
                       nullptr, qw, nullptr, nullptr, nullptr, M, N, K, 0, nullptr, false, P, tiles_n);
    return hipGetLastError();
}

}  // namespace svdq
