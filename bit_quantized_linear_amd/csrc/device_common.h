// Device-side helpers for the gfx950 (CDNA4) kernels of libsvdq.so:
// vector types, MFMA wrappers and the fixed rounding points.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svdq {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- MFMA (gfx950) ---------------------------------------------------------
// 32x32 outputs: lane l holds column (l % 32) and rows 8q + 4(l / 32) + t at
// element 4q + t (q, t in 0..3). 16x16 outputs: lane l holds column (l % 16)
// and rows 4(l / 16) + t at element t. A lane's A operand is one row and its
// B operand one column; A and B lanes of the same lane index carry the same
// K slots, so any K permutation applied identically to both leaves the
// product unchanged.

__device__ __forceinline__ i32x16 mfma_i8_32x32x32(i32x4 a, i32x4 b, i32x16 c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- conversions -----------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 -> packed bf16 (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950. Same result as f32_to_bf16_bits for every
// non-NaN input.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <class T>
__device__ __forceinline__ T bitcast(const void *p) {
    return *reinterpret_cast<const T *>(p);
}

// Nibble unpack for the INT4 path: 8 packed bytes (16 two's-complement
// nibbles, low nibble = even k) become 16 int8 values equal to 16 * code, in
// the order [k0, k2, ..., k14, k1, k3, ..., k15]. Shifting a nibble into the
// high half of its byte multiplies it by 16 exactly; the factor 16 * 16 = 256
// of a product is removed after the integer sum, exactly.
__device__ __forceinline__ void unpack_int4x16(uint32_t a, uint32_t b, uint32_t out[4]) {
    out[0] = (a << 4) & 0xF0F0F0F0u;
    out[1] = (b << 4) & 0xF0F0F0F0u;
    out[2] = a & 0xF0F0F0F0u;
    out[3] = b & 0xF0F0F0F0u;
}

// ---- Output tile store through LDS -----------------------------------------
// A block's (64 WN) (n) x 128 (m) output tile, held by WN x 2 waves (wn, wm)
// as 2 x 2 32x32 fp32 MFMA tiles each (lane: column m = wm 64 + im 32 +
// l % 32, rows n = wn 64 + in 32 + 8 qq + 4 (l / 32) + t), plus bias[n],
// rounded to bf16 (nearest even) or kept fp32, stored to Y [M][N] (row m, N
// contiguous). Stored straight from the MFMA layout, one instruction would
// write 16 bytes into each of 32 rows; staged through LDS instead, in two
// passes of 64 tokens (the waves of one wm row write, everyone stores), each
// 16-byte piece of a row segment of 128 WN (bf16) or 256 WN (fp32) bytes is
// stored by one lane, consecutive lanes along the row.
// Needs N % 8 == 0 and Y 16-byte aligned (16-byte pieces never straddle the
// end of a row), `lds` >= tile_store_lds_bytes(WN) bytes not in use by
// anyone, and all 128 WN threads of the block (it synchronizes).
constexpr int tile_store_lds_bytes(int WN) { return 64 * (256 * WN + 16); }
constexpr int kTileStoreLdsBytes = tile_store_lds_bytes(2);

template <int WN>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[2][2], uint8_t *lds, const uint16_t *__restrict__ bias,
                                           void *__restrict__ Y, bool y_f32, int M, int N, int m0, int n0, int wn,
                                           int wm, int tid) {
    constexpr int BN = 64 * WN;
    constexpr int THREADS = 128 * WN;
    const int lane = tid & 63, r32 = lane & 31, lh = lane >> 5;
    // row pitches padded by 8 / 16 bytes so that the 32 rows one write
    // instruction touches spread over the banks
    const int pitch = y_f32 ? 4 * BN + 16 : 2 * BN + 8;
    const int cpr = y_f32 ? BN / 4 : BN / 8;  // 16-byte pieces per row
    const int cols = y_f32 ? 4 : 8;           // columns per piece
    for (int p = 0; p < 2; ++p) {
        if (wm == p) {
#pragma unroll
            for (int in = 0; in < 2; ++in) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int nl = wn * 64 + in * 32 + 8 * qq + 4 * lh;
                    float bv[4] = {0.f, 0.f, 0.f, 0.f};
                    if (bias && n0 + nl < N) {
                        const u32x2 bb = *reinterpret_cast<const u32x2 *>(bias + n0 + nl);
                        bv[0] = bf16_bits_to_f32(bb[0] & 0xFFFFu);
                        bv[1] = bf16_bits_to_f32(bb[0] >> 16);
                        bv[2] = bf16_bits_to_f32(bb[1] & 0xFFFFu);
                        bv[3] = bf16_bits_to_f32(bb[1] >> 16);
                    }
#pragma unroll
                    for (int im = 0; im < 2; ++im) {
                        const int ml = im * 32 + r32;
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = acc[in][im][4 * qq + t] + bv[t];
                        if (y_f32)
                            *reinterpret_cast<f32x4 *>(lds + ml * pitch + nl * 4) = f32x4{v[0], v[1], v[2], v[3]};
                        else
                            *reinterpret_cast<u32x2 *>(lds + ml * pitch + nl * 2) =
                                u32x2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
                    }
                }
            }
        }
        __syncthreads();
        for (int c = tid; c < 64 * cpr; c += THREADS) {
            const int row = c / cpr, piece = c % cpr;
            const int m = m0 + 64 * p + row, n = n0 + piece * cols;
            if (m < M && n < N) {
                const uint8_t *src = lds + row * pitch + piece * 16;
                const u32x2 lo = *reinterpret_cast<const u32x2 *>(src);
                const u32x2 hi = *reinterpret_cast<const u32x2 *>(src + 8);
                uint8_t *dst = static_cast<uint8_t *>(Y) + ((size_t)m * N + n) * (y_f32 ? 4 : 2);
                *reinterpret_cast<u32x4 *>(dst) = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
        __syncthreads();
    }
}

__device__ __forceinline__ void store_tile_128x128(const f32x16 (&acc)[2][2], uint8_t *lds,
                                                   const uint16_t *__restrict__ bias, void *__restrict__ Y,
                                                   bool y_f32, int M, int N, int m0, int n0, int wn, int wm,
                                                   int tid) {
    store_tile<2>(acc, lds, bias, Y, y_f32, M, N, m0, n0, wn, wm, tid);
}

}  // namespace svdq
