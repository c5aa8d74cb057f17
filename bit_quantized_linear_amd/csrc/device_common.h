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
// A block's 128 (n) x 128 (m) output tile, held by 2 x 2 waves (wn, wm) as
// 2 x 2 32x32 fp32 MFMA tiles each (lane: column m = wm 64 + im 32 + l % 32,
// rows n = wn 64 + in 32 + 8 qq + 4 (l / 32) + t), plus bias[n], rounded to
// bf16 (nearest even) or kept fp32, stored to Y [M][N] (row m, N contiguous).
// Stored straight from the MFMA layout, one instruction would write 16 bytes
// into each of 32 rows; staged through LDS instead, each 16-byte piece of a
// row segment (256 bytes bf16, 512 bytes fp32) is stored by one lane,
// consecutive lanes along the row. A bf16 tile goes through LDS whole (every
// wave writes at once, one barrier); an fp32 tile in two passes of 64 tokens
// (the waves of one wm row write, everyone stores). Row pitches are padded
// by 8 / 16 bytes so that the 32 rows one write instruction touches spread
// over the banks.
// The bias comes from LDS as fp32 (stage_bias_128 at the start of the
// kernel, so no global load waits after the main loop).
// The LDS tile is held in two halves, lds_lo for the first half of the rows
// in LDS at a time and lds_hi for the second (two stage buffers of the
// caller, which need not be adjacent: kernels keep their stages in separate
// LDS variables so that the compiler can tell a stage being refilled from
// the one being read).
// Needs N % 8 == 0 and Y 16-byte aligned (16-byte pieces never straddle the
// end of a row), lds_lo and lds_hi >= kTileHalfLdsBytes bytes each, 16-byte
// aligned and not in use by anyone, and all 256 threads of the block (it
// synchronizes).
constexpr int kTileBf16Pitch = 2 * 128 + 8;
constexpr int kTileF32Pitch = 4 * 128 + 16;
constexpr int kTileHalfLdsBytes = 64 * kTileBf16Pitch > 32 * kTileF32Pitch ? 64 * kTileBf16Pitch
                                                                             : 32 * kTileF32Pitch;

// The block's 128 bias values bias[n0 .. n0 + 127] as fp32 into bias_s (16-
// byte aligned LDS), zero past N or without bias. A barrier between this and
// the first read makes them visible; the GEMM kernels call it before the
// barrier that precedes their main loop.
__device__ __forceinline__ void stage_bias_128(float *bias_s, const uint16_t *__restrict__ bias, int n0, int N,
                                               int tid) {
    if (tid < 128) bias_s[tid] = bias && n0 + tid < N ? bf16_bits_to_f32(bias[n0 + tid]) : 0.0f;
}

__device__ __forceinline__ void store_tile_128x128(const f32x16 (&acc)[2][2], uint8_t *lds_lo, uint8_t *lds_hi,
                                                   const float *bias_s, void *__restrict__ Y, bool y_f32, int M,
                                                   int N, int m0, int n0, int wn, int wm, int tid) {
    const int lane = tid & 63, r32 = lane & 31, lh = lane >> 5;
    if (!y_f32) {
#pragma unroll
        for (int in = 0; in < 2; ++in) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int nl = wn * 64 + in * 32 + 8 * qq + 4 * lh;
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(bias_s + nl);
#pragma unroll
                for (int im = 0; im < 2; ++im) {
                    // rows 0..63 (wm = 0) in the low half, 64..127 in the high
                    const int ml = im * 32 + r32;
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = acc[in][im][4 * qq + t] + bv[t];
                    *reinterpret_cast<u32x2 *>((wm ? lds_hi : lds_lo) + ml * kTileBf16Pitch + nl * 2) =
                        u32x2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
                }
            }
        }
        __syncthreads();
        uint16_t *y = static_cast<uint16_t *>(Y);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i;  // 128 rows x 16 pieces
            const int row = c >> 4, piece = c & 15;
            const int m = m0 + row, n = n0 + piece * 8;
            if (m < M && n < N) {
                // rows are 8-byte aligned (264-byte pitch): two 8-byte reads
                const uint8_t *src = (row < 64 ? lds_lo + row * kTileBf16Pitch
                                               : lds_hi + (row - 64) * kTileBf16Pitch) + piece * 16;
                const u32x2 lo = *reinterpret_cast<const u32x2 *>(src);
                const u32x2 hi = *reinterpret_cast<const u32x2 *>(src + 8);
                *reinterpret_cast<u32x4 *>(y + (size_t)m * N + n) = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
        return;
    }
    float *y = static_cast<float *>(Y);
    for (int p = 0; p < 2; ++p) {
        if (p) __syncthreads();  // the first pass's reads are done
        if (wm == p) {
#pragma unroll
            for (int in = 0; in < 2; ++in) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int nl = wn * 64 + in * 32 + 8 * qq + 4 * lh;
                    const f32x4 bv = *reinterpret_cast<const f32x4 *>(bias_s + nl);
#pragma unroll
                    for (int im = 0; im < 2; ++im) {
                        // pass rows 0..31 (im = 0) in the low half, 32..63 in the high
                        f32x4 v;
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = acc[in][im][4 * qq + t] + bv[t];
                        *reinterpret_cast<f32x4 *>((im ? lds_hi : lds_lo) + r32 * kTileF32Pitch + nl * 4) = v;
                    }
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i;  // 64 rows x 32 pieces
            const int row = c >> 5, piece = c & 31;
            const int m = m0 + 64 * p + row, n = n0 + piece * 4;
            if (m < M && n < N)
                *reinterpret_cast<u32x4 *>(y + (size_t)m * N + n) = *reinterpret_cast<const u32x4 *>(
                    (row < 32 ? lds_lo + row * kTileF32Pitch : lds_hi + (row - 32) * kTileF32Pitch) + piece * 16);
        }
    }
}

// The same for a 128 (features) x 64 (tokens) tile whose waves (wn, wm)
// hold features wn * 64 .. wn * 64 + 63 of tokens wm * 32 .. wm * 32 + 31
// (one 32-token slice each): a bf16 tile goes through LDS whole (64 rows),
// an fp32 tile in two passes of 32 tokens (the waves of one wm write,
// everyone stores). lds needs kTile64LdsBytes bytes, 16-byte aligned and
// not in use by anyone; the rest as for store_tile_128x128.
constexpr int kTile64LdsBytes = 64 * kTileBf16Pitch > 32 * kTileF32Pitch ? 64 * kTileBf16Pitch
                                                                           : 32 * kTileF32Pitch;

__device__ __forceinline__ void store_tile_128x64(const f32x16 (&acc)[2][1], uint8_t *lds, const float *bias_s,
                                                  void *__restrict__ Y, bool y_f32, int M, int N, int m0, int n0,
                                                  int wn, int wm, int tid) {
    const int lane = tid & 63, r32 = lane & 31, lh = lane >> 5;
    if (!y_f32) {
#pragma unroll
        for (int in = 0; in < 2; ++in) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int nl = wn * 64 + in * 32 + 8 * qq + 4 * lh;
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(bias_s + nl);
                const int ml = wm * 32 + r32;
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = acc[in][0][4 * qq + t] + bv[t];
                *reinterpret_cast<u32x2 *>(lds + ml * kTileBf16Pitch + nl * 2) =
                    u32x2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
            }
        }
        __syncthreads();
        uint16_t *y = static_cast<uint16_t *>(Y);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;  // 64 rows x 16 pieces
            const int row = c >> 4, piece = c & 15;
            const int m = m0 + row, n = n0 + piece * 8;
            if (m < M && n < N) {
                const uint8_t *src = lds + row * kTileBf16Pitch + piece * 16;
                const u32x2 lo = *reinterpret_cast<const u32x2 *>(src);
                const u32x2 hi = *reinterpret_cast<const u32x2 *>(src + 8);
                *reinterpret_cast<u32x4 *>(y + (size_t)m * N + n) = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
        return;
    }
    float *y = static_cast<float *>(Y);
    for (int p = 0; p < 2; ++p) {
        if (p) __syncthreads();  // the first pass's reads are done
        if (wm == p) {
#pragma unroll
            for (int in = 0; in < 2; ++in) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int nl = wn * 64 + in * 32 + 8 * qq + 4 * lh;
                    const f32x4 bv = *reinterpret_cast<const f32x4 *>(bias_s + nl);
                    f32x4 v;
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = acc[in][0][4 * qq + t] + bv[t];
                    *reinterpret_cast<f32x4 *>(lds + r32 * kTileF32Pitch + nl * 4) = v;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;  // 32 rows x 32 pieces
            const int row = c >> 5, piece = c & 31;
            const int m = m0 + 32 * p + row, n = n0 + piece * 4;
            if (m < M && n < N)
                *reinterpret_cast<u32x4 *>(y + (size_t)m * N + n) =
                    *reinterpret_cast<const u32x4 *>(lds + row * kTileF32Pitch + piece * 16);
        }
    }
}

}  // namespace svdq
