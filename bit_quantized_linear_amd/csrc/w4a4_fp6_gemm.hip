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
// Block tile 128 (n) x 128 (m), 4 waves as 2 x 2, wave tile 64 x 64 (2 x 2
// MFMA tiles of 32 x 32); two blocks fit a CU. One LDS stage holds two
// groups (K = 128): 128 x 96 code bytes of each operand and 2 x 256 scales.
// Global loads are buffer loads with per-thread offsets computed once; rows
// beyond M or N fall outside the buffer and read as zero, so the tails need
// no branches. Each thread moves the same six 16-byte chunks per stage.
// Staged rows are padded to 56 bytes so that 32 lanes reading 8 bytes from 32
// consecutive rows touch distinct LDS banks. Stages are double buffered with
// one barrier per stage, the next stage's loads in flight during the MFMAs.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace svdq {

namespace {

constexpr int BN = 128;
constexpr int BM = 128;
constexpr int THREADS = 256;
constexpr int KG = 2;            // groups per LDS stage
constexpr int ROW6 = 56;         // LDS stride of one staged 48-byte row
constexpr int GB = 48;           // code bytes per row and group
constexpr int E8M0_X8 = 127 + 3; // MFMA block scale 2^3
constexpr uint32_t kOob = 0x80000000u;  // an offset past any buffer

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

struct Stage6 {
    uint8_t a[KG][BN * ROW6];
    uint8_t b[KG][BM * ROW6];
    float sa[KG][BN];
    float sb[KG][BM];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ float buf_load4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// 24 bytes (the 32 codes of lane half lh) of one staged row
__device__ __forceinline__ i32x8 frag6(const uint8_t *row_base, int lh) {
    const uint8_t *p = row_base + 24 * lh;
    const u32x2 x0 = *reinterpret_cast<const u32x2 *>(p);
    const u32x2 x1 = *reinterpret_cast<const u32x2 *>(p + 8);
    const u32x2 x2 = *reinterpret_cast<const u32x2 *>(p + 16);
    return i32x8{(int)x0[0], (int)x0[1], (int)x1[0], (int)x1[1], (int)x2[0], (int)x2[1], 0, 0};
}

template <bool kLinear>
__global__ __launch_bounds__(THREADS, 2) void w4a4_fp6_kernel(
    const uint8_t *__restrict__ qx, const float *__restrict__ sx, const uint16_t *__restrict__ T,
    const uint8_t *__restrict__ qw, const float *__restrict__ sw, const uint16_t *__restrict__ l2t,
    const uint16_t *__restrict__ bias, int M, int N, int K, int rank, void *__restrict__ Y, bool y_f32,
    int32_t *__restrict__ Pout, int tiles_n) {
    __shared__ Stage6 stage[2];

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int n0 = tile_n * BN;
    const int m0 = tile_m * BM;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int G = K / 64;
    const int S = (G + KG - 1) / KG;
    const uint32_t R = (uint32_t)K / 4 * 3;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw, (uint32_t)N * R);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(qx, (uint32_t)M * R);

    // this thread's three chunks of each operand per stage: chunk c = tid +
    // 256 i covers row c / 6, 16-byte part (c % 6) of the stage's 96 bytes
    uint32_t goff_a[3], goff_b[3], lds_a[3], lds_b[3];
    int slot[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int c = tid + THREADS * i;
        const int row = c / 6, p = c - 6 * (c / 6);
        const int j = p / 3, part = p - 3 * (p / 3);
        slot[i] = j;
        goff_a[i] = (uint32_t)(n0 + row) * R + (uint32_t)(j * GB + part * 16);
        goff_b[i] = (uint32_t)(m0 + row) * R + (uint32_t)(j * GB + part * 16);
        lds_a[i] = (uint32_t)(j * BN * ROW6 + row * ROW6 + part * 16);
        lds_b[i] = (uint32_t)(j * BM * ROW6 + row * ROW6 + part * 16);
    }
    // scales: waves 0-1 stage sx (token side), waves 2-3 sw (weight side)
    const int sel = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int sj = tid & 127;
    const int sL = sel ? N : M;
    const int sbase = sel ? n0 : m0;
    const bool s_ok = sbase + sj < sL;
    __amdgpu_buffer_rsrc_t rs = make_rsrc(sel ? (const void *)sw : (const void *)sx, (uint32_t)G * (uint32_t)sL * 4u);

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

    u32x4 ra[3], rb[3];
    float rsv[KG];
    auto load_stage = [&](int s) {
        const int g0 = s * KG;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const bool ok = g0 + slot[i] < G;
            const uint32_t adv = (uint32_t)g0 * GB;
            ra[i] = buf_load16(rw, ok ? goff_a[i] + adv : kOob);
            rb[i] = buf_load16(rx, ok ? goff_b[i] + adv : kOob);
        }
        if constexpr (kLinear) {
#pragma unroll
            for (int q = 0; q < KG; ++q) {
                const bool ok = s_ok && g0 + q < G;
                const uint32_t off = ((uint32_t)(g0 + q) * (uint32_t)sL + (uint32_t)(sbase + sj)) * 4u;
                rsv[q] = buf_load4f(rs, ok ? off : kOob);
            }
        }
    };
    auto store_stage = [&](Stage6 &st) {
        uint8_t *a = &st.a[0][0];
        uint8_t *bb = &st.b[0][0];
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            *reinterpret_cast<u32x2 *>(a + lds_a[i]) = u32x2{ra[i][0], ra[i][1]};
            *reinterpret_cast<u32x2 *>(a + lds_a[i] + 8) = u32x2{ra[i][2], ra[i][3]};
            *reinterpret_cast<u32x2 *>(bb + lds_b[i]) = u32x2{rb[i][0], rb[i][1]};
            *reinterpret_cast<u32x2 *>(bb + lds_b[i] + 8) = u32x2{rb[i][2], rb[i][3]};
        }
        if constexpr (kLinear) {
#pragma unroll
            for (int q = 0; q < KG; ++q) {
                if (sel)
                    st.sa[q][sj] = rsv[q];
                else
                    st.sb[q][sj] = rsv[q];
            }
        }
    };

    load_stage(0);
    store_stage(stage[0]);
    __syncthreads();

    for (int s = 0; s < S; ++s) {
        const Stage6 &cur = stage[s & 1];
        if (s + 1 < S) load_stage(s + 1);
        const int ng = min(KG, G - s * KG);
#pragma unroll
        for (int q = 0; q < KG; ++q) {
            if (q >= ng) break;
            i32x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = frag6(cur.a[q] + (wn * 64 + i * 32 + r32) * ROW6, lh);
                b[i] = frag6(cur.b[q] + (wm * 64 + i * 32 + r32) * ROW6, lh);
            }
#pragma unroll
            for (int in = 0; in < 2; ++in) {
#pragma unroll
                for (int im = 0; im < 2; ++im) {
                    const f32x16 P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a[in], b[im], zero16, 2, 2, 0, E8M0_X8, 0, E8M0_X8);
                    if constexpr (kLinear) {
                        const float sxm = cur.sb[q][wm * 64 + im * 32 + r32];
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) {
                            const f32x4 s4 = *reinterpret_cast<const f32x4 *>(&cur.sa[q][wn * 64 + in * 32 + 8 * qq + 4 * lh]);
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                acc[in][im][4 * qq + t] = fmaf(sxm * s4[t], P[4 * qq + t], acc[in][im][4 * qq + t]);
                        }
                    } else {
                        const int g = s * KG + q;
                        const int m = m0 + wm * 64 + im * 32 + r32;
                        if (m < M) {
#pragma unroll
                            for (int qq = 0; qq < 4; ++qq) {
                                const int n = n0 + wn * 64 + in * 32 + 8 * qq + 4 * lh;
                                if (n < N) {
                                    i32x4 v;
#pragma unroll
                                    for (int t = 0; t < 4; ++t) v[t] = (int)P[4 * qq + t];
                                    *reinterpret_cast<i32x4 *>(Pout + ((size_t)g * M + m) * N + n) = v;
                                }
                            }
                        }
                    }
                }
            }
        }
        if (s + 1 < S) store_stage(stage[(s + 1) & 1]);
        __syncthreads();
    }

    if constexpr (kLinear) {
        for (int kk = 0; kk < rank; kk += 16) {
            bf16x8 la[2], lb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int n = n0 + wn * 64 + i * 32 + r32;
                const int m = m0 + wm * 64 + i * 32 + r32;
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
            for (int qq = 0; qq < 4; ++qq) {
                const int n = n0 + wn * 64 + in * 32 + 8 * qq + 4 * lh;
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
                    const int m = m0 + wm * 64 + im * 32 + r32;
                    if (m >= M) continue;
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = acc[in][im][4 * qq + t] + bv[t];
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
