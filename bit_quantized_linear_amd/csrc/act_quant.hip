// Fused activation quantization for the SVDQuant W4A4 linear, and the
// per-channel calibration statistic for smoothing.
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
// paragraph -- activations are quantized to 4 bits after their outliers have
// been moved into the weights, and a 16-bit low-rank branch runs beside the
// 4-bit product. One pass over X produces the packed INT4 codes, their group
// scales and the branch's down-projection T = X L1s.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"
#include "quant_common.h"

namespace svdq {

namespace {

constexpr int kActWaves = 8;   // waves per block; they split the K groups
constexpr int kActRows = 16;   // token rows per block (one 16x16 MFMA row tile)

// One block owns 16 token rows and a range of K groups (all of K, or a
// 1 / gridDim.y share when the launcher splits K across blocks so that
// small batches still fill the chip); wave w takes the range's groups w,
// w + 8, ... . Lane l holds row (l % 16) and the 16 consecutive channels
// [64 g + 16 (l / 16), +16) of group g: two 128-bit loads of X. The four
// lanes of a row meet through two cross-lane max steps for the group absmax.
// For the branch, the lane's 16 channels feed two 16x16x32 bf16 MFMAs per
// rank tile (8 channels each); B comes from l1t with the same channel
// mapping. The 8 waves' fp32 partial T tiles are summed in wave order through
// LDS; with K split, each block stores its fp32 partial and a second kernel
// sums the partials in K order, so T is deterministic either way.
// E2M1 code of q (|q| < 8): nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to
// the even mantissa (rintf rounds half to even, and in each binade the even
// multiple of the quantum is the even mantissa), saturating at 6; bit 3 is
// the sign; a value that rounds to zero is +0.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
    const float m = fabsf(q);
    const float r = m < 2.0f ? rintf(2.0f * m) * 0.5f : (m < 4.0f ? rintf(m) : fminf(6.0f, 2.0f * rintf(0.5f * m)));
    const int c = r < 2.0f ? (int)(2.0f * r) : (r < 4.0f ? (int)r + 2 : (int)(0.5f * r) + 4);
    return (uint32_t)c | ((c != 0 && q < 0.0f) ? 8u : 0u);
}

// MX shared exponent of a block: floor(log2 amax) - 2 clamped to [-127, 127],
// -127 for amax == 0, read off the fp32 bit pattern.
__device__ __forceinline__ int mx_exponent(float amax) {
    const uint32_t b = __float_as_uint(amax);
    if (b == 0u) return -127;
    const int ex = (int)(b >> 23);
    const int fl = ex != 0 ? ex - 127 : (31 - __clz((int)b)) - 149;  // floor(log2 amax), subnormals too
    return min(127, max(-127, fl - 2));
}

enum ActFmt { kInt4 = 0, kFp6 = 1, kMx = 2 };

// kFmt: kInt4 / kFp6 write INT4 codes with fp32 group scales (sx [K/64, M]);
// kMx writes MXFP4 codes with E8M0 block scales (sx points to u8 [K/32][ld]).
template <int kFmt, int RT>
__global__ __launch_bounds__(kActWaves * 64) void quantize_act_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ smooth,
    const uint16_t *__restrict__ l1t, int M, int K, int rank,
    uint8_t *__restrict__ qx, void *__restrict__ sx_out, int sx_ld, uint16_t *__restrict__ T,
    float *__restrict__ tpart) {
    constexpr int kRT = RT > 0 ? RT : 1;  // rank tiles held (rank / 16, at least one array slot)
    __shared__ float red[kActWaves][kActRows][16 * kRT];
    __shared__ double rcp[kActWaves][SVDQ_GROUP];  // per wave: 1/s of its current group's channels

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane & 15;
    const int quad = lane >> 4;
    const int m0 = blockIdx.x * kActRows;
    const int m = m0 + row;
    const bool row_ok = m < M;
    const int G = K / SVDQ_GROUP;
    const int g_lo = (int)(blockIdx.y * G / gridDim.y), g_hi = (int)((blockIdx.y + 1) * G / gridDim.y);
    constexpr int rtiles = RT;

    f32x4 tacc[kRT];
#pragma unroll
    for (int i = 0; i < kRT; ++i) tacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // X and the smoothing factor of the wave's next group are loaded one
    // group ahead, so their latency overlaps the current group's work
    u32x4 nxa = {0u, 0u, 0u, 0u}, nxb = {0u, 0u, 0u, 0u};
    float ns = 1.0f;
    auto load_next = [&](int g) {
        if (g < g_hi) {
            if (row_ok) {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(X + (size_t)m * K + g * SVDQ_GROUP + quad * 16);
                nxa = p[0];
                nxb = p[1];
            }
            ns = smooth[g * SVDQ_GROUP + lane];
        }
    };
    load_next(g_lo + wave);
    for (int g = g_lo + wave; g < g_hi; g += kActWaves) {
        const int kb = g * SVDQ_GROUP + quad * 16;
        const u32x4 xa = nxa, xb = nxb;
        const float sg = ns;
        load_next(g + kActWaves);
        // 1/s of the group's 64 channels, one fp64 division per lane, shared
        // through this wave's slice of LDS
        rcp[wave][lane] = 1.0 / (double)sg;
        __builtin_amdgcn_wave_barrier();
        const double *rq = &rcp[wave][quad * 16];
        float xb16[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w0 = (i < 2) ? xa[2 * i] : xb[2 * (i - 2)];
            const uint32_t w1 = (i < 2) ? xa[2 * i + 1] : xb[2 * (i - 2) + 1];
            xb16[4 * i + 0] = bf16_bits_to_f32(w0 & 0xFFFFu);
            xb16[4 * i + 1] = bf16_bits_to_f32(w0 >> 16);
            xb16[4 * i + 2] = bf16_bits_to_f32(w1 & 0xFFFFu);
            xb16[4 * i + 3] = bf16_bits_to_f32(w1 >> 16);
        }
        // X_hat = fp32(X / s), the IEEE quotient, computed as
        // fp32(double(x) * fp64(1/s)): see quotient_fp32 for why it is exact
        float xh[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) xh[t] = quotient_fp32(xb16[t], rq[t]);
        __builtin_amdgcn_wave_barrier();
        // bamax: the 32-channel half of the group (lanes of quads 0-1 or 2-3),
        // amax: the whole group
        float bamax = 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) bamax = fmaxf(bamax, fabsf(xh[t]));
        bamax = fmaxf(bamax, __shfl_xor(bamax, 16));
        float amax = fmaxf(bamax, __shfl_xor(bamax, 32));
        if (amax < kTinyGroup) {
            // below the range quotient_fp32 covers: plain IEEE divisions
            // (all four lanes of the row take this branch together)
            const f32x4 *sp = reinterpret_cast<const f32x4 *>(smooth + kb);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 s4 = sp[i];
#pragma unroll
                for (int t = 0; t < 4; ++t) xh[4 * i + t] = xb16[4 * i + t] / s4[t];
            }
            bamax = 0.0f;
#pragma unroll
            for (int t = 0; t < 16; ++t) bamax = fmaxf(bamax, fabsf(xh[t]));
            bamax = fmaxf(bamax, __shfl_xor(bamax, 16));
            amax = fmaxf(bamax, __shfl_xor(bamax, 32));
        }
        const float scale = amax / 7.0f;
        // code = RNE(fp32(x_hat / scale)), the quotient again via fp64
        const double rscale = scale != 0.0f ? 1.0 / (double)scale : 0.0;
        if constexpr (kFmt == kMx) {
            // MXFP4: the lane's 16 channels lie in block 2g + quad / 2; its
            // codes are x_hat / 2^e (exact, a power of two: 2^-e is a normal
            // fp32 for every clamped e) in E2M1, 8 bytes at byte 8 (quad % 2)
            // of the row's 16-byte half h = quad / 2 of the group
            const int e = mx_exponent(bamax);
            const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
            uint32_t packed[2] = {0u, 0u};
#pragma unroll
            for (int t = 0; t < 16; ++t) packed[t >> 3] |= e2m1_code(xh[t] * inv) << (4 * (t & 7));
            if (row_ok) {
                const int b0 = m & ~127;
                const int nb = min(128, M - b0);
                uint8_t *dst = qx + (size_t)b0 * (K / 2) + (size_t)g * nb * 32 + (size_t)(quad >> 1) * nb * 16 +
                               (size_t)(m - b0) * 16 + 8 * (quad & 1);
                *reinterpret_cast<u32x2 *>(dst) = u32x2{packed[0], packed[1]};
                if ((quad & 1) == 0)
                    static_cast<uint8_t *>(sx_out)[(size_t)(2 * g + (quad >> 1)) * sx_ld + m] = (uint8_t)(e + 127);
            }
        } else if constexpr (kFmt == kInt4) {
            // INT4 container: two's-complement nibbles, low nibble = even k
            uint32_t packed[2] = {0u, 0u};
            if (scale != 0.0f) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const uint32_t nib = (uint32_t)int4_code(xh[t], rscale) & 0xFu;
                    packed[t >> 3] |= nib << (4 * (t & 7));
                }
            }
            if (row_ok)
                *reinterpret_cast<u32x2 *>(qx + (size_t)m * (K / 2) + kb / 2) = u32x2{packed[0], packed[1]};
        } else {
            // FP6 container: each code c as FP6 E2M3 of value c / 8 (sign bit,
            // zero exponent, 3-bit magnitude), 6-bit fields packed LSB-first
            // into the 24 bytes H_h of its half h = quad / 2; this lane's 16
            // codes are bytes [12 (quad % 2), +12) of H_h. In the row's 48
            // bytes of the group, H_h[0:16] sits at 16 h and H_h[16:24] at
            // 32 + 8 h.
            uint32_t w[3] = {0u, 0u, 0u};
            if (scale != 0.0f) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    const uint32_t v = fp6_field(int4_code(xh[t], rscale));
                    const int bit = 6 * t;
                    w[bit >> 5] |= v << (bit & 31);
                    if ((bit & 31) > 26) w[(bit >> 5) + 1] |= v >> (32 - (bit & 31));
                }
            }
            if (row_ok) {
                // blocks of 128 rows; inside a block, group g's rows follow
                // one another (48 bytes each) after the block's earlier groups
                const int b0 = m & ~127;
                const int nb = min(128, M - b0);
                uint8_t *grp = qx + (size_t)b0 * (K / 4 * 3) + ((size_t)g * nb + (m - b0)) * 48;
                const int h = quad >> 1;
                uint32_t *d0, *d1, *d2;
                if ((quad & 1) == 0) {
                    d0 = reinterpret_cast<uint32_t *>(grp + 16 * h);
                    d1 = d0 + 1;
                    d2 = d0 + 2;
                } else {
                    d0 = reinterpret_cast<uint32_t *>(grp + 16 * h + 12);
                    d1 = reinterpret_cast<uint32_t *>(grp + 32 + 8 * h);
                    d2 = d1 + 1;
                }
                *d0 = w[0];
                *d1 = w[1];
                *d2 = w[2];
            }
        }
        if constexpr (kFmt != kMx)
            if (row_ok && quad == 0) static_cast<float *>(sx_out)[(size_t)g * M + m] = scale;

        // low-rank down-projection on raw X (1/s folded into L1s)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, s == 0 ? xa : xb);
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                if (rt < rtiles) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(
                        l1t + (size_t)(rt * 16 + row) * K + kb + 8 * s);
                    tacc[rt] = mfma_bf16_16x16x32(a, b, tacc[rt]);
                }
            }
        }
    }

    if (rtiles == 0) return;
    // 16x16 output: lane holds column (lane % 16) = rank index within the
    // tile, rows 4 (lane / 16) + t
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        if (rt < rtiles) {
#pragma unroll
            for (int t = 0; t < 4; ++t) red[wave][4 * quad + t][rt * 16 + row] = tacc[rt][t];
        }
    }
    __syncthreads();
    const int elems = kActRows * rank;
    for (int e = threadIdx.x; e < elems; e += blockDim.x) {
        const int r = e / rank;
        const int j = e - r * rank;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kActWaves; ++w) v += red[w][r][j];
        if (m0 + r < M) {
            if (gridDim.y == 1)
                T[(size_t)(m0 + r) * rank + j] = (uint16_t)f32_to_bf16_bits(v);
            else
                tpart[((size_t)blockIdx.y * M + m0 + r) * rank + j] = v;
        }
    }
}

// Running per-channel max |X[m, k]| on the fp32 bit patterns (an unsigned
// max on the magnitudes' bit patterns is order-independent, hence
// deterministic). Block: 64 chunks of 8 channels x 4 row lanes, 64 rows.
constexpr int kAbsRows = 64;

__global__ __launch_bounds__(256) void channel_absmax_kernel(const uint16_t *__restrict__ X, int M,
                                                             int K, float *__restrict__ absmax) {
    __shared__ uint32_t red[4][64][8];
    const int chunk = blockIdx.x * 64 + (threadIdx.x & 63);
    const int rl = threadIdx.x >> 6;
    const int k0 = chunk * 8;
    const int mbeg = blockIdx.y * kAbsRows;
    const int mend = min(M, mbeg + kAbsRows);
    uint32_t mx[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (k0 < K) {
        for (int m = mbeg + rl; m < mend; m += 4) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(X + (size_t)m * K + k0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mx[2 * i] = max(mx[2 * i], (v[i] & 0x7FFFu) << 16);
                mx[2 * i + 1] = max(mx[2 * i + 1], (v[i] >> 16 & 0x7FFFu) << 16);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) red[rl][threadIdx.x & 63][t] = mx[t];
    __syncthreads();
    if (rl == 0 && k0 < K) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            uint32_t v = max(max(red[0][threadIdx.x][t], red[1][threadIdx.x][t]),
                             max(red[2][threadIdx.x][t], red[3][threadIdx.x][t]));
            atomicMax(reinterpret_cast<unsigned int *>(absmax + k0 + t), v);
        }
    }
}

}  // namespace

template <int RT>
static void launch_act_rt(dim3 grid, hipStream_t stream, int fmt, const uint16_t *X, const float *smooth,
                          const uint16_t *l1t, int M, int K, int rank, uint8_t *qx, void *sx, int sx_ld,
                          uint16_t *T, float *tpart) {
    if (fmt == kFp6)
        hipLaunchKernelGGL((quantize_act_kernel<kFp6, RT>), grid, dim3(kActWaves * 64), 0, stream, X, smooth,
                           l1t, M, K, rank, qx, sx, sx_ld, T, tpart);
    else if (fmt == kMx)
        hipLaunchKernelGGL((quantize_act_kernel<kMx, RT>), grid, dim3(kActWaves * 64), 0, stream, X, smooth,
                           l1t, M, K, rank, qx, sx, sx_ld, T, tpart);
    else
        hipLaunchKernelGGL((quantize_act_kernel<kInt4, RT>), grid, dim3(kActWaves * 64), 0, stream, X, smooth,
                           l1t, M, K, rank, qx, sx, sx_ld, T, tpart);
}

// How many blocks share the K range of one 16-row tile: the largest divisor
// d of the group count that leaves every wave whole groups (G / d a multiple
// of 8, the waves per block) and keeps the grid within 4 blocks per compute
// unit, or within 8 when each block still has 4 groups per wave. More parts
// balance the grid better but add T partials to write and sum (measured at
// M = 4608: 3 parts best at K = 3072, 6 at K = 12288).
int act_k_parts(int M, int K) {
    const int64_t blocks = (M + kActRows - 1) / kActRows;
    const int G = K / SVDQ_GROUP;
    int kp = 1;
    for (int d = 2; d <= G / kActWaves; ++d) {
        if (G % d != 0 || (G / d) % kActWaves != 0) continue;
        if (blocks * d <= 1024 || (blocks * d <= 2048 && G / d >= 4 * kActWaves)) kp = d;
    }
    return kp;
}

size_t act_workspace_size(int M, int K, int rank) {
    if (M <= 0 || K <= 0 || rank <= 0) return 0;
    const int kp = act_k_parts(M, K);
    return kp > 1 ? (size_t)kp * (size_t)M * (size_t)rank * sizeof(float) : 0;
}

// Without a workspace for T's partials the K range is split only when there
// is no T (rank 0).
static hipError_t launch_act(const uint16_t *X, const float *smooth, const uint16_t *l1t, int M, int K,
                             int rank, int fmt, uint8_t *qx, void *sx, int sx_ld, uint16_t *T, float *workspace,
                      hipStream_t stream) {
    const int kp = (rank == 0 || workspace) ? act_k_parts(M, K) : 1;
    float *tpart = kp > 1 && rank ? workspace : nullptr;
    const dim3 grid((M + kActRows - 1) / kActRows, kp);
    switch (rank / 16) {  // rank % 16 == 0 and rank <= 64 are checked by the caller
        case 0: launch_act_rt<0>(grid, stream, fmt, X, smooth, l1t, M, K, rank, qx, sx, sx_ld, T, tpart); break;
        case 1: launch_act_rt<1>(grid, stream, fmt, X, smooth, l1t, M, K, rank, qx, sx, sx_ld, T, tpart); break;
        case 2: launch_act_rt<2>(grid, stream, fmt, X, smooth, l1t, M, K, rank, qx, sx, sx_ld, T, tpart); break;
        case 3: launch_act_rt<3>(grid, stream, fmt, X, smooth, l1t, M, K, rank, qx, sx, sx_ld, T, tpart); break;
        default: launch_act_rt<4>(grid, stream, fmt, X, smooth, l1t, M, K, rank, qx, sx, sx_ld, T, tpart); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !tpart) return e;
    return launch_tpart_reduce(tpart, kp, M, rank, T, stream);
}

hipError_t launch_quantize_act(const uint16_t *X, const float *smooth, const uint16_t *l1t, int M,
                               int K, int rank, int qfmt, uint8_t *qx, float *sx, uint16_t *T,
                               float *workspace, hipStream_t stream) {
    return launch_act(X, smooth, l1t, M, K, rank, qfmt == SVDQ_QFMT_FP6 ? kFp6 : kInt4, qx, sx, M, T, workspace,
                      stream);
}

hipError_t launch_mx_quantize_act(const uint16_t *X, const float *smooth, const uint16_t *l1t, int M,
                                  int K, int rank, uint8_t *qx, uint8_t *ux, uint16_t *T, float *workspace,
                                  hipStream_t stream) {
    return launch_act(X, smooth, l1t, M, K, rank, kMx, qx, ux, (int)mx_scale_ld(M), T, workspace, stream);
}

hipError_t launch_channel_absmax(const uint16_t *X, int M, int K, float *absmax,
                                 hipStream_t stream) {
    const int chunks = (K + 7) / 8;
    const dim3 grid((chunks + 63) / 64, (M + kAbsRows - 1) / kAbsRows);
    hipLaunchKernelGGL(channel_absmax_kernel, grid, dim3(256), 0, stream, X, M, K, absmax);
    return hipGetLastError();
}

}  // namespace svdq
