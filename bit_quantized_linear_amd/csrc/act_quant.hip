// Fused activation quantization for the SVDQuant W4A4 linear, and the
// per-channel calibration statistic for smoothing.
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
// paragraph -- activations are quantized to 4 bits after their outliers have
// been moved into the weights, and a 16-bit low-rank branch runs beside the
// 4-bit product. One pass over X produces the packed INT4 codes, their group
// scales and the branch's down-projection T = X L1s.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "internal.h"
#include "quant_common.h"

namespace svdq {

namespace {

constexpr int kActWaves = 4;   // waves per block, one 16-row tile each
constexpr int kActRows = 16;   // token rows per wave (one 16x16 MFMA row tile)

// MX shared exponent of a block: floor(log2 amax) - 2 clamped to [-127, 127],
// -127 for amax == 0, read off the fp32 bit pattern.
__device__ __forceinline__ int mx_exponent(float amax) {
    const uint32_t b = __float_as_uint(amax);
    if (b == 0u) return -127;
    const int ex = (int)(b >> 23);
    const int fl = ex != 0 ? ex - 127 : (31 - __clz((int)b)) - 149;  // floor(log2 amax), subnormals too
    return min(127, max(-127, fl - 2));
}

// Eight E2M1 codes, one per nibble, with the sign of each zero code cleared:
// the conversion keeps the sign of a negative value that rounds to zero,
// while a zero code is +0 (a nibble's sign bit 3 survives only where its
// magnitude bits 0-2 are not all zero).
__device__ __forceinline__ uint32_t clear_negative_zero_fp4(uint32_t w) {
    const uint32_t mag = w & 0x77777777u;
    const uint32_t nonzero = (mag + 0x77777777u) & 0x88888888u;  // bit 3 of each nibble: magnitude != 0
    return mag | (w & nonzero);
}

enum ActFmt { kInt4 = 0, kFp6 = 1, kMx = 2 };

// One block of 4 waves owns 64 token rows (16 per wave) and a range of K
// groups (all of K, or a 1 / gridDim.y share when the launcher splits K
// across blocks so that the chip fills); the waves walk the range's groups
// in step. Lane l holds row (l % 16) of its wave's tile and the 16
// consecutive channels [64 g + 16 (l / 16), +16) of group g: two 128-bit
// loads of X, issued one group ahead. The four lanes of a row meet through
// two cross-lane max steps for the group absmax. What every wave needs of a
// group -- the L1s slice [rank][64 channels] and 1/s of the 64 channels --
// is staged once per block in LDS (double buffered, one barrier per group):
// the slice is loaded into registers one group ahead and written after the
// barrier, and one wave (the waves take turns) loads the group's smoothing
// factors and computes their fp64 reciprocals. For the branch, the lane's 16
// channels feed two 16x16x32 bf16 MFMAs per rank tile (8 channels each),
// with B from the staged slice in the same channel mapping; each wave keeps
// its own rows' T, so no reduction across waves is needed. With K split,
// each block stores its fp32 partial and a second kernel sums the partials
// in K order, so T is deterministic either way.
// kFmt: kInt4 / kFp6 write INT4 codes with fp32 group scales (sx [K/64, M]);
// kMx writes MXFP4 codes with E8M0 block scales (sx points to u8 [K/32][ld]).
template <int kFmt, int RT>
__global__ __launch_bounds__(kActWaves * 64) void quantize_act_kernel(
    const uint16_t *__restrict__ X, const float *__restrict__ smooth,
    const uint16_t *__restrict__ l1t, int M, int K, int rank,
    uint8_t *__restrict__ qx, void *__restrict__ sx_out, int sx_ld, uint16_t *__restrict__ T,
    float *__restrict__ tpart) {
    constexpr int kRT = RT > 0 ? RT : 1;  // rank tiles held (rank / 16, at least one array slot)
    constexpr int kLsPitch = 2 * SVDQ_GROUP + 16;  // bytes per rank row of a staged L1s slice (padded)
    // per group, shared by the block's waves: the L1s slice [rank][64 channels]
    // and 1/s of the 64 channels, double buffered
    __shared__ __attribute__((aligned(16))) uint8_t ls[2][16 * kRT * kLsPitch];
    __shared__ double rcp[2][SVDQ_GROUP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int row = lane & 15;
    const int quad = lane >> 4;
    const int m0 = blockIdx.x * (kActWaves * kActRows) + wave * kActRows;
    const int m = m0 + row;
    const bool row_ok = m < M;
    const int G = K / SVDQ_GROUP;
    const int g_lo = (int)(blockIdx.y * G / gridDim.y), g_hi = (int)((blockIdx.y + 1) * G / gridDim.y);
    constexpr int rtiles = RT;

    f32x4 tacc[kRT];
#pragma unroll
    for (int i = 0; i < kRT; ++i) tacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // a group's L1s slice is rank rows of 128 bytes, 8 chunks of 16 bytes
    // each; thread t loads chunks t, t + 256 (one group ahead, into
    // registers) and writes them into the staged slice after the group's
    // barrier. The smoothing factors of a group are loaded by one wave (the
    // waves take turns), which also computes their reciprocals.
    constexpr int kPer = (16 * kRT * 8 + kActWaves * 64 - 1) / (kActWaves * 64);
    u32x4 lnext[kPer];
    float snext = 1.0f;
    auto ls_load = [&](int g) __attribute__((always_inline)) {
        if (g < g_hi) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int c = tid + kActWaves * 64 * j;
                if (c < rank * 8)
                    lnext[j] = *reinterpret_cast<const u32x4 *>(l1t + (size_t)(c >> 3) * K + g * SVDQ_GROUP +
                                                                (c & 7) * 8);
            }
            if (wave == (g & (kActWaves - 1))) snext = smooth[g * SVDQ_GROUP + lane];
        }
    };
    auto ls_store = [&](int g, int b) __attribute__((always_inline)) {
        if (g < g_hi) {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int c = tid + kActWaves * 64 * j;
                if (c < rank * 8) *reinterpret_cast<u32x4 *>(&ls[b][(c >> 3) * kLsPitch + (c & 7) * 16]) = lnext[j];
            }
            if (wave == (g & (kActWaves - 1))) rcp[b][lane] = 1.0 / (double)snext;
        }
    };

    // X of the wave's next group is loaded one group ahead
    u32x4 nxa = {0u, 0u, 0u, 0u}, nxb = {0u, 0u, 0u, 0u};
    auto load_next = [&](int g) __attribute__((always_inline)) {
        if (g < g_hi && row_ok) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(X + (size_t)m * K + g * SVDQ_GROUP + quad * 16);
            nxa = p[0];
            nxb = p[1];
        }
    };
    load_next(g_lo);
    ls_load(g_lo);
    ls_store(g_lo, 0);
    __syncthreads();
    int buf = 0;
    for (int g = g_lo; g < g_hi; ++g, buf ^= 1) {
        const int kb = g * SVDQ_GROUP + quad * 16;
        const u32x4 xa = nxa, xb = nxb;
        load_next(g + 1);
        ls_load(g + 1);
        const double *rq = &rcp[buf][quad * 16];
        // X_hat = fp32(X / s), the IEEE quotient, computed as
        // fp32(double(x) * fp64(1/s)): see quotient_fp32 for why it is exact
        float xh[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w0 = (i < 2) ? xa[2 * i] : xb[2 * (i - 2)];
            const uint32_t w1 = (i < 2) ? xa[2 * i + 1] : xb[2 * (i - 2) + 1];
            xh[4 * i + 0] = quotient_fp32(bf16_bits_to_f32(w0 & 0xFFFFu), rq[4 * i + 0]);
            xh[4 * i + 1] = quotient_fp32(bf16_bits_to_f32(w0 >> 16), rq[4 * i + 1]);
            xh[4 * i + 2] = quotient_fp32(bf16_bits_to_f32(w1 & 0xFFFFu), rq[4 * i + 2]);
            xh[4 * i + 3] = quotient_fp32(bf16_bits_to_f32(w1 >> 16), rq[4 * i + 3]);
        }
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
                const uint32_t w0 = (i < 2) ? xa[2 * i] : xb[2 * (i - 2)];
                const uint32_t w1 = (i < 2) ? xa[2 * i + 1] : xb[2 * (i - 2) + 1];
                xh[4 * i + 0] = bf16_bits_to_f32(w0 & 0xFFFFu) / s4[0];
                xh[4 * i + 1] = bf16_bits_to_f32(w0 >> 16) / s4[1];
                xh[4 * i + 2] = bf16_bits_to_f32(w1 & 0xFFFFu) / s4[2];
                xh[4 * i + 3] = bf16_bits_to_f32(w1 >> 16) / s4[3];
            }
            bamax = 0.0f;
#pragma unroll
            for (int t = 0; t < 16; ++t) bamax = fmaxf(bamax, fabsf(xh[t]));
            bamax = fmaxf(bamax, __shfl_xor(bamax, 16));
            amax = fmaxf(bamax, __shfl_xor(bamax, 32));
        }
        if constexpr (kFmt == kMx) {
            // MXFP4: the lane's 16 channels lie in block 2g + quad / 2; its
            // codes are E2M1 of x_hat / 2^e (x_hat * 2^-e is exact: 2^-e is a
            // normal fp32 for every clamped e, and a product that underflows
            // is far below the smallest nonzero code). The conversion rounds
            // to nearest, ties to the even mantissa, saturating at 6; its
            // operands fill the low and the high nibble of the byte it
            // writes. 8 bytes at byte 8 (quad % 2) of the row's 16-byte half
            // h = quad / 2 of the group.
            const int e = mx_exponent(bamax);
            const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
            uint32_t packed[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t w = 0u;
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * h + 0] * inv, xh[8 * h + 1] * inv, 1.0f, 0);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * h + 2] * inv, xh[8 * h + 3] * inv, 1.0f, 1);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * h + 4] * inv, xh[8 * h + 5] * inv, 1.0f, 2);
                w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, xh[8 * h + 6] * inv, xh[8 * h + 7] * inv, 1.0f, 3);
                packed[h] = clear_negative_zero_fp4(w);
            }
            if (row_ok) {
                const int b0 = m & ~127;
                const int nb = min(128, M - b0);
                uint8_t *dst = qx + (size_t)b0 * (K / 2) + (size_t)g * nb * 32 + (size_t)(quad >> 1) * nb * 16 +
                               (size_t)(m - b0) * 16 + 8 * (quad & 1);
                *reinterpret_cast<u32x2 *>(dst) = u32x2{packed[0], packed[1]};
                if ((quad & 1) == 0)
                    static_cast<uint8_t *>(sx_out)[(size_t)(2 * g + (quad >> 1)) * sx_ld + m] = (uint8_t)(e + 127);
            }
        } else {
            // scale = fp32(amax / 7): amax is 0 or at least 2^-100 here, so
            // the fp64 reciprocal product is the IEEE quotient (quotient_fp32)
            const float scale = quotient_fp32(amax, kRcp7);
            // code = RNE(fp32(x_hat / scale)), the quotient again via fp64
            const double rscale = scale != 0.0f ? 1.0 / (double)scale : 0.0;
            if constexpr (kFmt == kInt4) {
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
                // FP6 container: each code c as FP6 E2M3 of value c / 8 (sign
                // bit, zero exponent, 3-bit magnitude), 6-bit fields packed
                // LSB-first into the 24 bytes H_h of its half h = quad / 2;
                // this lane's 16 codes are bytes [12 (quad % 2), +12) of H_h.
                // In the row's 48 bytes of the group, H_h[0:16] sits at 16 h
                // and H_h[16:24] at 32 + 8 h.
                float v[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) v[t] = fp6_value(xh[t], rscale);
                uint32_t w[3];
                pack_fp6_16(v, w);
                if (row_ok) {
                    // blocks of 128 rows; inside a block, group g's rows
                    // follow one another (48 bytes each) after the block's
                    // earlier groups
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
            if (row_ok && quad == 0) static_cast<float *>(sx_out)[(size_t)g * M + m] = scale;
        }

        // low-rank down-projection on raw X (1/s folded into L1s); B from
        // the staged slice, same channel mapping as the lane's X
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, s == 0 ? xa : xb);
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                if (rt < rtiles) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8 *>(
                        &ls[buf][(rt * 16 + row) * kLsPitch + (quad * 16 + 8 * s) * 2]);
                    tacc[rt] = mfma_bf16_16x16x32(a, b, tacc[rt]);
                }
            }
        }
        // the next group's slice and 1/s into the other buffer (read by no
        // one since the barrier that ended the previous group); the barrier
        // makes them visible and ends this group's reads of `buf`
        ls_store(g + 1, buf ^ 1);
        __syncthreads();
    }

    if (rtiles == 0) return;
    // 16x16 output: lane holds column (lane % 16) = rank index within the
    // tile, rows 4 (lane / 16) + t of the wave's 16 rows
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        if (rt < rtiles) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int mm = m0 + 4 * quad + t;
                if (mm < M) {
                    if (gridDim.y == 1)
                        T[(size_t)mm * rank + rt * 16 + row] = (uint16_t)f32_to_bf16_bits(tacc[rt][t]);
                    else
                        tpart[((size_t)blockIdx.y * M + mm) * rank + rt * 16 + row] = tacc[rt][t];
                }
            }
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

// How many blocks share the K range of one 64-row block (K parts): enough
// to give the GPU about 2048 blocks of four waves, but no fewer than six
// groups per block (each group costs the block a barrier and a staged L1s
// slice, and each part a [M][rank] fp32 slice of partial sums), and at most
// 131072 / M parts, so that the partials of every accepted shape (rank <=
// 64) fit the 32 MiB scratch of the allocation-free pass. Measured at
// M = 4608: 8 parts best at K = 3072 (6 groups each), 24-32 at K = 12288;
// at M = 32760, K = 5120: 2-4 parts.
int act_k_parts(int M, int K) {
    if (M <= 0) return 1;
    const int64_t row_blocks = (M + kActWaves * kActRows - 1) / (kActWaves * kActRows);
    const int G = K / SVDQ_GROUP;
    int64_t kp = std::min<int64_t>(G / 6, 2048 / row_blocks);
    kp = std::min<int64_t>(kp, 131072 / M);
    return (int)std::max<int64_t>(1, kp);
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
    const dim3 grid((M + kActWaves * kActRows - 1) / (kActWaves * kActRows), kp);
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

// Scratch of the allocation-free activation pass (svdq_quantize_act_noalloc):
// the fp32 partial sums of T, [parts][M][rank], when K is split across
// blocks. act_k_parts keeps parts x M <= 131072, so the partials never exceed
// 131072 x 64 x 4 bytes = 32 MiB. Every element the reduction reads is
// written by the same call first, so nothing needs clearing; calls that
// overlap on one device share this array and race.
static __device__ __align__(256) float scratch[kActScratchBytes / sizeof(float)];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kScratchDevices];
}  // namespace

hipError_t act_scratch_pointer(float **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        // the array's device address on this device (its name in host code
        // is only a host-side handle)
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<float *>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
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
