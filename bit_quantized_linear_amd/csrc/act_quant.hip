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

namespace svdq {

namespace {

constexpr int kActWaves = 8;   // waves per block; they split the K groups
constexpr int kActRows = 16;   // token rows per block (one 16x16 MFMA row tile)

// One block owns 16 token rows and walks all K groups; wave w takes groups
// w, w + 8, ... . Lane l holds row (l % 16) and the 16 consecutive channels
// [64 g + 16 (l / 16), +16) of group g: two 128-bit loads of X. The four
// lanes of a row meet through two cross-lane max steps for the group absmax.
// For the branch, the lane's 16 channels feed two 16x16x32 bf16 MFMAs per
// rank tile (8 channels each); B comes from l1t with the same channel
// mapping. The 8 waves' fp32 partial T tiles are summed in wave order through
// LDS, so T is deterministic.
template <bool kFp6>
__global__ __launch_bounds__(kActWaves * 64) void quantize_act_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ smooth,
    const uint16_t *__restrict__ l1t, int M, int K, int rank,
    uint8_t *__restrict__ qx, float *__restrict__ sx, uint16_t *__restrict__ T) {
    __shared__ float red[kActWaves][kActRows][SVDQ_MAX_RANK];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane & 15;
    const int quad = lane >> 4;
    const int m0 = blockIdx.x * kActRows;
    const int m = m0 + row;
    const bool row_ok = m < M;
    const int G = K / SVDQ_GROUP;
    const int rtiles = rank >> 4;

    f32x4 tacc[SVDQ_MAX_RANK / 16];
#pragma unroll
    for (int i = 0; i < SVDQ_MAX_RANK / 16; ++i) tacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int g = wave; g < G; g += kActWaves) {
        const int kb = g * SVDQ_GROUP + quad * 16;
        u32x4 xa = {0u, 0u, 0u, 0u}, xb = {0u, 0u, 0u, 0u};
        if (row_ok) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(X + (size_t)m * K + kb);
            xa = p[0];
            xb = p[1];
        }
        const f32x4 *sp = reinterpret_cast<const f32x4 *>(smooth + kb);
        float xh[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 s4 = sp[i];
            const uint32_t w0 = (i < 2) ? xa[2 * i] : xb[2 * (i - 2)];
            const uint32_t w1 = (i < 2) ? xa[2 * i + 1] : xb[2 * (i - 2) + 1];
            // X_hat = fp32(X / s): IEEE division, round to nearest even
            xh[4 * i + 0] = bf16_bits_to_f32(w0 & 0xFFFFu) / s4[0];
            xh[4 * i + 1] = bf16_bits_to_f32(w0 >> 16) / s4[1];
            xh[4 * i + 2] = bf16_bits_to_f32(w1 & 0xFFFFu) / s4[2];
            xh[4 * i + 3] = bf16_bits_to_f32(w1 >> 16) / s4[3];
        }
        float amax = 0.0f;
#pragma unroll
        for (int t = 0; t < 16; ++t) amax = fmaxf(amax, fabsf(xh[t]));
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float scale = amax / 7.0f;

        if constexpr (!kFp6) {
            // INT4 container: two's-complement nibbles, low nibble = even k
            uint32_t packed[2] = {0u, 0u};
            if (scale != 0.0f) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float q = rintf(xh[t] / scale);  // round half to even
                    q = fminf(7.0f, fmaxf(-7.0f, q));
                    const uint32_t nib = (uint32_t)((int)q) & 0xFu;
                    packed[t >> 3] |= nib << (4 * (t & 7));
                }
            }
            if (row_ok)
                *reinterpret_cast<u32x2 *>(qx + (size_t)m * (K / 2) + kb / 2) = u32x2{packed[0], packed[1]};
        } else {
            // FP6 container: each code c as FP6 E2M3 of value c / 8 (sign bit,
            // zero exponent, 3-bit magnitude), 6-bit fields packed LSB-first
            // into the 24 bytes H_h of its half h = quad / 2; this lane's 16
            // codes are bytes [12 (quad % 2), +12) of H_h. In the group's 48
            // bytes, H_h[0:16] sits at 16 h and H_h[16:24] at 32 + 8 h.
            uint32_t w[3] = {0u, 0u, 0u};
            if (scale != 0.0f) {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float q = rintf(xh[t] / scale);  // round half to even
                    q = fminf(7.0f, fmaxf(-7.0f, q));
                    const int qi = (int)q;
                    const uint32_t v = (qi < 0 ? 0x20u : 0u) | (uint32_t)(qi < 0 ? -qi : qi);
                    const int bit = 6 * t;
                    w[bit >> 5] |= v << (bit & 31);
                    if ((bit & 31) > 26) w[(bit >> 5) + 1] |= v >> (32 - (bit & 31));
                }
            }
            if (row_ok) {
                uint8_t *grp = qx + (size_t)m * (K / 4 * 3) + (size_t)g * 48;
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
        if (row_ok && quad == 0) sx[(size_t)g * M + m] = scale;

        // low-rank down-projection on raw X (1/s folded into L1s)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, s == 0 ? xa : xb);
#pragma unroll
            for (int rt = 0; rt < SVDQ_MAX_RANK / 16; ++rt) {
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
    for (int rt = 0; rt < SVDQ_MAX_RANK / 16; ++rt) {
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
        if (m0 + r < M) T[(size_t)(m0 + r) * rank + j] = (uint16_t)f32_to_bf16_bits(v);
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

hipError_t launch_quantize_act(const uint16_t *X, const float *smooth, const uint16_t *l1t, int M,
                               int K, int rank, int qfmt, uint8_t *qx, float *sx, uint16_t *T,
                               hipStream_t stream) {
    const dim3 grid((M + kActRows - 1) / kActRows);
    if (qfmt == SVDQ_QFMT_FP6)
        hipLaunchKernelGGL(quantize_act_kernel<true>, grid, dim3(kActWaves * 64), 0, stream, X, smooth, l1t,
                           M, K, rank, qx, sx, T);
    else
        hipLaunchKernelGGL(quantize_act_kernel<false>, grid, dim3(kActWaves * 64), 0, stream, X, smooth, l1t,
                           M, K, rank, qx, sx, T);
    return hipGetLastError();
}

hipError_t launch_channel_absmax(const uint16_t *X, int M, int K, float *absmax,
                                 hipStream_t stream) {
    const int chunks = (K + 7) / 8;
    const dim3 grid((chunks + 63) / 64, (M + kAbsRows - 1) / kAbsRows);
    hipLaunchKernelGGL(channel_absmax_kernel, grid, dim3(256), 0, stream, X, M, K, absmax);
    return hipGetLastError();
}

}  // namespace svdq
