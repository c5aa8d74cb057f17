// Integer-MFMA GEMM core shared by the W4A4 and W8A8 linears of libsvdq.so.
//
// C^T tile = A . B^T with A = weight rows (output columns n, K contiguous)
// and B = activation rows (tokens m, K contiguous), both staged through LDS
// as int8 and multiplied on gfx950 v_mfma_i32_32x32x32_i8 with int32
// accumulation. One K step is 64 elements: one INT4 group (2 MFMAs of K 32).
//
//  - Block: 256 threads = 4 waves as 2 (n) x 2 (m); block tile 128 n x 128 m;
//    wave tile 64 x 64 = 2 x 2 MFMA tiles of 32 x 32.
//  - Main loop: global -> registers (one 128-bit load per operand per thread
//    for INT4, two for INT8) -> INT4 nibbles unpacked to int8 -> LDS, double
//    buffered with one barrier per K step; the next step's global loads are
//    issued before the current step's MFMAs.
//  - LDS rows are padded from 64 to 80 bytes so the 16-byte operand reads of
//    32 consecutive rows spread over all banks.
//  - Tails: rows of A beyond N and of B beyond M are zero-filled on load and
//    never stored.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace svdq {

constexpr int kTileN = 128;
constexpr int kTileM = 128;
constexpr int kGemmThreads = 256;
constexpr int kKStep = 64;
constexpr int kLdsRow = 80;  // bytes per staged row (64 data + 16 pad)

struct GemmStage {
    uint8_t a[kTileN * kLdsRow];
    uint8_t b[kTileM * kLdsRow];
    float sa[kTileN];  // per-step weight-side scales (INT4 only)
    float sb[kTileM];  // per-step activation-side scales (INT4 only)
};

// Operand fetch for one K step. INT4: each thread owns 16 packed bytes of one
// row (row = tid / 2, half = tid % 2 -> packed bytes [16 half, +16) of the
// step's 32). INT8: 32 bytes of one row (two 128-bit loads).
template <bool kInt4>
struct StepRegs {
    u32x4 a[kInt4 ? 1 : 2];
    u32x4 b[kInt4 ? 1 : 2];
    float sc;  // one scale (threads 0..127 activation side, 128..255 weight side)
};

template <bool kInt4, bool kScales>
__device__ __forceinline__ void load_step(StepRegs<kInt4> &r, const uint8_t *__restrict__ A,
                                          const uint8_t *__restrict__ B, const float *__restrict__ sA,
                                          const float *__restrict__ sB, int n0, int m0, int N, int M,
                                          int K, int step) {
    const int tid = threadIdx.x;
    const int row = tid >> 1;
    const int half = tid & 1;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if constexpr (kInt4) {
        const size_t ld = (size_t)K / 2;
        const size_t off = (size_t)step * 32 + half * 16;
        r.a[0] = (n0 + row < N) ? *reinterpret_cast<const u32x4 *>(A + (size_t)(n0 + row) * ld + off) : zero;
        r.b[0] = (m0 + row < M) ? *reinterpret_cast<const u32x4 *>(B + (size_t)(m0 + row) * ld + off) : zero;
        r.sc = 0.0f;
        if constexpr (kScales) {
            if (tid < kTileM) {
                r.sc = (m0 + tid < M) ? sB[(size_t)step * M + m0 + tid] : 0.0f;
            } else {
                const int j = tid - kTileM;
                r.sc = (n0 + j < N) ? sA[(size_t)step * N + n0 + j] : 0.0f;
            }
        }
    } else {
        const size_t ld = (size_t)K;
        const size_t off = (size_t)step * 64 + half * 32;
        if (n0 + row < N) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(A + (size_t)(n0 + row) * ld + off);
            r.a[0] = p[0];
            r.a[1] = p[1];
        } else {
            r.a[0] = zero;
            r.a[1] = zero;
        }
        if (m0 + row < M) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(B + (size_t)(m0 + row) * ld + off);
            r.b[0] = p[0];
            r.b[1] = p[1];
        } else {
            r.b[0] = zero;
            r.b[1] = zero;
        }
        r.sc = 0.0f;
    }
}

// Registers -> LDS. Each row's 64 int8 values sit as four 16-byte chunks;
// chunk c holds the K slice [16 c, 16 c + 16) of the step (INT4: in the
// unpacked order [even k..., odd k...] of that slice).
template <bool kInt4>
__device__ __forceinline__ void store_step(GemmStage &st, const StepRegs<kInt4> &r) {
    const int tid = threadIdx.x;
    const int row = tid >> 1;
    const int half = tid & 1;
    uint8_t *da = st.a + row * kLdsRow + half * 32;
    uint8_t *db = st.b + row * kLdsRow + half * 32;
    if constexpr (kInt4) {
        uint32_t u[4];
        unpack_int4x16(r.a[0][0], r.a[0][1], u);
        *reinterpret_cast<u32x4 *>(da) = u32x4{u[0], u[1], u[2], u[3]};
        unpack_int4x16(r.a[0][2], r.a[0][3], u);
        *reinterpret_cast<u32x4 *>(da + 16) = u32x4{u[0], u[1], u[2], u[3]};
        unpack_int4x16(r.b[0][0], r.b[0][1], u);
        *reinterpret_cast<u32x4 *>(db) = u32x4{u[0], u[1], u[2], u[3]};
        unpack_int4x16(r.b[0][2], r.b[0][3], u);
        *reinterpret_cast<u32x4 *>(db + 16) = u32x4{u[0], u[1], u[2], u[3]};
        if (tid < kTileM)
            st.sb[tid] = r.sc;
        else
            st.sa[tid - kTileM] = r.sc;
    } else {
        *reinterpret_cast<u32x4 *>(da) = r.a[0];
        *reinterpret_cast<u32x4 *>(da + 16) = r.a[1];
        *reinterpret_cast<u32x4 *>(db) = r.b[0];
        *reinterpret_cast<u32x4 *>(db + 16) = r.b[1];
    }
}

// One K step of MFMAs for this wave's 2 x 2 tiles: P[in][im] += A . B^T.
__device__ __forceinline__ void mma_step(const GemmStage &st, int wn, int wm, i32x16 P[2][2]) {
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
        const int c = 2 * kh + lh;
        i32x4 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a[i] = *reinterpret_cast<const i32x4 *>(st.a + (wn * 64 + i * 32 + r32) * kLdsRow + 16 * c);
            b[i] = *reinterpret_cast<const i32x4 *>(st.b + (wm * 64 + i * 32 + r32) * kLdsRow + 16 * c);
        }
#pragma unroll
        for (int in = 0; in < 2; ++in)
#pragma unroll
            for (int im = 0; im < 2; ++im) P[in][im] = mfma_i8_32x32x32(a[in], b[im], P[in][im]);
    }
}

}  // namespace svdq
