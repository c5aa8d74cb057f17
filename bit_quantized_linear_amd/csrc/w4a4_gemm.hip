// The SVDQuant W4A4 linear on the INT4 container: INT4 x INT4 GEMM with
// per-group scaling, fused with the 16-bit low-rank up-projection and the
// bias.
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru), method
// paragraph (4-bit weights x 4-bit activations with a 16-bit low-rank branch)
// and "Nunchaku Lite" paragraph (svdq_w4a4 layers for the attention and MLP
// projections, INT4 variant). Grouped INT4 format: "Diffusion Compiler"
// README, "Compiler" bullet.
//
//   P[g, m, n] = sum_{k in g} qx[m, k] qw[n, k]          (int32, exact)
//   acc[m, n] += fp32(sx[g, m] sw[g, n]) * P[g, m, n]     (fp32, g ascending)
//   y = acc + T L2 + bias  ->  bf16 (nearest even) or fp32
//
// The container holds one row's 64 codes of a group in 32 bytes, code k in
// nibble k % 2 of byte k / 2 (two's complement). A nibble moved to the high
// half of a byte reads as the int8 16 * code, so one AND (odd codes) or a
// shift and an AND (even codes) turn four bytes of nibbles into two int8
// MFMA operands; v_mfma_i32_32x32x32_i8 on the even codes, then on the odd
// ones, sums the whole group. The K order inside a group does not matter as
// long as both operands use the same one: the sum is exact in int32. The
// MFMA thus returns 256 * P, so the main loop accumulates
// acc' = sum_g fp32(sx sw) (256 P) -- 256 times the fp32 accumulator of the
// formula above at every step, since a power-of-two factor commutes with
// each rounding -- and acc = acc' / 256 is taken once before the low-rank
// branch is added. The scale products come from the matrix core: the
// two-block fp32 MFMA with K = 1 returns sw[n] sx[m] for two 32 x 32 tiles in
// the lane layout of their partials, each rounded once as a VALU multiply
// rounds it. The vector ALU converts each partial to fp32 and does one FMA
// per output element and group.
//
// Block tile 128 (n) x 128 (m), 4 waves as 2 x 2, wave tile 64 x 64 (2 x 2
// MFMA tiles of 32 x 32). One LDS stage holds two groups: per operand and
// group 128 rows x 32 bytes (4 KB) and the groups' 2 x 128 scales, copied
// straight from global memory to LDS (buffer_load ... lds, 16 bytes per
// lane). Load i of a group tile covers rows 32 i .. 32 i + 31: lane l takes
// row 32 i + l % 32 and the row's bytes 16 (l / 32) .. +15, and lands at
// 1024 i + 16 l, so a lane's MFMA operand (row r, byte half h) is one 16-byte
// read at 1024 (r / 32) + 512 h + 16 (r % 32) and the 64 lanes of a read
// cover 1 KB without bank conflicts. Rows past the end of an operand read
// zeros (the whole offset is in the per-lane offset, so the range check sees
// it) and feed only outputs that are never stored. Stages are double
// buffered in two LDS variables (so the compiler does not make the reads of
// one wait for the loads into the other), with one barrier per stage.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace svdq {

namespace {

enum class W4Epilogue { kLinear, kPartials };

constexpr int kI4BN = 128;
constexpr int kI4BM = 128;
constexpr int kI4Threads = 256;
constexpr int kI4KG = 2;                // groups per LDS stage
constexpr int kI4GB = 32;               // container bytes per row and group
constexpr int kI4Tile = 128 * kI4GB;    // one group of 128 rows: 4 KB

typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef __attribute__((address_space(3))) void lds_void_t;

struct Stage4 {
    uint8_t a[kI4KG * kI4Tile];  // [group][32-row block][byte half][row][16 bytes]
    uint8_t b[kI4KG * kI4Tile];
    float sa[kI4KG][kI4BN];
    float sb[kI4KG][kI4BM];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc4(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes of nibbles (32 codes) -> the int8 operands 16 * code of the even
// codes (low nibbles) and of the odd codes (high nibbles)
__device__ __forceinline__ void unpack_nibbles(const u32x4 &w, i32x4 &even, i32x4 &odd) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        even[d] = (int)((w[d] << 4) & 0xF0F0F0F0u);
        odd[d] = (int)(w[d] & 0xF0F0F0F0u);
    }
}

template <W4Epilogue kEpi>
__global__ __launch_bounds__(kI4Threads, 3) void w4a4_int4_kernel(
    const uint8_t *__restrict__ qx, const float *__restrict__ sx, const uint16_t *__restrict__ T,
    const uint8_t *__restrict__ qw, const float *__restrict__ sw, const uint16_t *__restrict__ l2t,
    const uint16_t *__restrict__ bias, int M, int N, int K, int rank, void *__restrict__ Y, bool y_f32,
    int32_t *__restrict__ Pout, int tiles_n) {
    constexpr bool kLinear = kEpi == W4Epilogue::kLinear;
    __shared__ __attribute__((aligned(16))) Stage4 st0;
    __shared__ __attribute__((aligned(16))) Stage4 st1;

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int n0 = tile_n * kI4BN;
    const int m0 = tile_m * kI4BM;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int G = K / 64;
    const int S = (G + kI4KG - 1) / kI4KG;
    const uint32_t RB = (uint32_t)K / 2;  // container bytes per row

    const __amdgpu_buffer_rsrc_t rw = rsrc4(qw, (uint32_t)N * RB);
    const __amdgpu_buffer_rsrc_t rx = rsrc4(qx, (uint32_t)M * RB);
    const __amdgpu_buffer_rsrc_t rsw = rsrc4(sw, (uint32_t)G * (uint32_t)N * 4u);
    const __amdgpu_buffer_rsrc_t rsx = rsrc4(sx, (uint32_t)G * (uint32_t)M * 4u);

    // Per stage the block issues 16 operand loads of 1 KB: wave w loads the
    // tile of operand w / 2 (0: weights, 1: tokens) and group w % 2 of the
    // stage, four loads of 32 rows each. The scales of a side are two runs
    // of 4 bytes per row (one per group) in memory and one [2][128] array in
    // LDS: with four rows per lane one 16-byte load per side puts both in
    // place (wave 2 the weight side, wave 3 the token side). That needs the
    // runs to start on 16 bytes, i.e. a row count that is a multiple of 4 (N
    // always is); for M % 4 != 0 the token side takes four 4-byte loads, one
    // per group and 64-row half, by waves 2 and 3.
    const int op_w = wave >> 1, q_w = wave & 1;
    const uint32_t lane_off = (uint32_t)((op_w ? m0 : n0) + r32) * RB + 16u * (uint32_t)lh;
    const bool sx16 = (M & 3) == 0;
    const int s_side = wave == 2;
    const bool s_lane = wave >= 2;
    const int s_slot = lane >> 5;
    const uint32_t s_off = (uint32_t)((s_side ? n0 : m0) + 4 * r32) * 4u;

    auto issue_stage = [&](int s, Stage4 &st) __attribute__((always_inline)) {
        const int g = s * kI4KG + q_w;
        if (g < G) {
            uint8_t *dst = (op_w ? st.b : st.a) + q_w * kI4Tile;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(op_w ? rx : rw, (lds_void_t *)(dst + i * 1024), 16,
                                                         lane_off + (uint32_t)i * 32u * RB + (uint32_t)g * 32u, 0,
                                                         0, 0);
        }
        if constexpr (kLinear) {
            if (s_lane && (sx16 || s_side)) {
                // a group past G lies past the end of the buffer: zeros, never read
                const uint32_t L = s_side ? (uint32_t)N : (uint32_t)M;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(s_side ? rsw : rsx,
                                                         (lds_void_t *)(s_side ? &st.sa[0][0] : &st.sb[0][0]), 16,
                                                         (uint32_t)(s * kI4KG + s_slot) * L * 4u + s_off, 0, 0, 0);
            }
            if (!sx16 && wave >= 2) {
                const int slot = wave - 2, gs = s * kI4KG + slot;
#pragma unroll
                for (int half = 0; half < 2; ++half)
                    if (gs < G)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rsx, (lds_void_t *)(st.sb[slot] + half * 64), 4,
                            ((uint32_t)gs * (uint32_t)M + (uint32_t)(m0 + half * 64 + lane)) * 4u, 0, 0, 0);
            }
        }
    };

    // this lane's operand reads within a staged group tile
    const int a_off = (wn * 2) * 1024 + lh * 512 + r32 * 16;  // + in * 1024
    const int b_off = (wm * 2) * 1024 + lh * 512 + r32 * 16;  // + im * 1024

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const i32x16 izero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const f32x32 zero32 = {};

    __shared__ __attribute__((aligned(16))) float bias_s[kI4BN];
    if constexpr (kLinear) stage_bias_128(bias_s, bias, n0, N, tid);
    issue_stage(0, st0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    auto run_stage = [&](int s, const Stage4 &cur, Stage4 &nxt) __attribute__((always_inline)) {
        if (s + 1 < S) issue_stage(s + 1, nxt);
        const int ng = min(kI4KG, G - s * kI4KG);
#pragma unroll
        for (int q = 0; q < kI4KG; ++q) {
            if (q >= ng) break;
            i32x4 ae[2], ao[2];
#pragma unroll
            for (int in = 0; in < 2; ++in)
                unpack_nibbles(*reinterpret_cast<const u32x4 *>(cur.a + q * kI4Tile + a_off + in * 1024), ae[in],
                               ao[in]);
            float swv = 0.0f;
            if constexpr (kLinear) swv = cur.sa[q][wn * 64 + lane];
#pragma unroll
            for (int im = 0; im < 2; ++im) {
                // keep the scheduler from hoisting the next slice's operands
                // (and their registers) into this one
                __builtin_amdgcn_sched_barrier(0);
                i32x4 be, bo;
                unpack_nibbles(*reinterpret_cast<const u32x4 *>(cur.b + q * kI4Tile + b_off + im * 1024), be, bo);
                if constexpr (kLinear) {
                    const float sxv = cur.sb[q][wm * 64 + im * 32 + r32];
                    __builtin_amdgcn_s_setprio(1);
                    const f32x32 C = __builtin_amdgcn_mfma_f32_32x32x1f32(swv, sxv, zero32, 0, 0, 0);
                    i32x16 P0 = mfma_i8_32x32x32(ae[0], be, izero);
                    P0 = mfma_i8_32x32x32(ao[0], bo, P0);
                    i32x16 P1 = mfma_i8_32x32x32(ae[1], be, izero);
                    P1 = mfma_i8_32x32x32(ao[1], bo, P1);
                    __builtin_amdgcn_s_setprio(0);
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[0][im][e] = fmaf(C[e], (float)P0[e], acc[0][im][e]);
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[1][im][e] = fmaf(C[16 + e], (float)P1[e], acc[1][im][e]);
                } else {
                    // rows of a 32 x 32 partial are weight rows n = 8 qq + 4 lh + t,
                    // its column the token m = r32
                    const int g = s * kI4KG + q;
                    const int m = m0 + wm * 64 + im * 32 + r32;
#pragma unroll
                    for (int in = 0; in < 2; ++in) {
                        i32x16 P = mfma_i8_32x32x32(ae[in], be, izero);
                        P = mfma_i8_32x32x32(ao[in], bo, P);
                        if (m < M) {
#pragma unroll
                            for (int qq = 0; qq < 4; ++qq) {
                                const int n = n0 + wn * 64 + in * 32 + 8 * qq + 4 * lh;
                                if (n < N) {
                                    i32x4 v;
#pragma unroll
                                    for (int t = 0; t < 4; ++t) v[t] = P[4 * qq + t] >> 8;
                                    *reinterpret_cast<i32x4 *>(Pout + ((size_t)g * M + m) * N + n) = v;
                                }
                            }
                        }
                    }
                }
            }
        }
        // the next stage's loads must have landed before anyone reads them,
        // and everyone must be done with this stage before it is refilled
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int s = 0; s < S; s += 2) {
        run_stage(s, st0, st1);
        if (s + 1 < S) run_stage(s + 1, st1, st0);
    }

    if constexpr (kLinear) {
        // acc = acc' / 256 (exact while acc is a normal fp32 number; a result
        // in the subnormal range is rounded once more, by at most half of
        // 2^-149)
#pragma unroll
        for (int in = 0; in < 2; ++in)
#pragma unroll
            for (int im = 0; im < 2; ++im)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[in][im][e] *= 1.0f / 256.0f;
        // low-rank up-projection: C^T += L2^T-rows (A, weight side) x T-rows
        // (B, token side) on bf16 MFMA, K = rank in slices of 16
        for (int kk = 0; kk < rank; kk += 16) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int n = n0 + wn * 64 + i * 32 + r32;
                const int m = m0 + wm * 64 + i * 32 + r32;
                u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
                if (n < N) va = *reinterpret_cast<const u32x4 *>(l2t + (size_t)n * rank + kk + 8 * lh);
                if (m < M) vb = *reinterpret_cast<const u32x4 *>(T + (size_t)m * rank + kk + 8 * lh);
                a[i] = __builtin_bit_cast(bf16x8, va);
                b[i] = __builtin_bit_cast(bf16x8, vb);
            }
#pragma unroll
            for (int in = 0; in < 2; ++in)
#pragma unroll
                for (int im = 0; im < 2; ++im) acc[in][im] = mfma_bf16_32x32x16(a[in], b[im], acc[in][im]);
        }
        // every load has landed and been read: the stage buffers hold the
        // output tile on its way out
        static_assert(sizeof(Stage4) >= kTileHalfLdsBytes, "LDS too small for the output tile");
        store_tile_128x128(acc, reinterpret_cast<uint8_t *>(&st0), reinterpret_cast<uint8_t *>(&st1), bias_s, Y,
                           y_f32, M, N, m0, n0, wn, wm, tid);
    }
}

}  // namespace

hipError_t launch_w4a4_linear(const uint8_t *qx, const float *sx, const uint16_t *T,
                              const uint8_t *qw, const float *sw, const uint16_t *l2t,
                              const uint16_t *bias, int M, int N, int K, int rank, void *Y,
                              bool y_f32, hipStream_t stream) {
    const int tiles_n = (N + kI4BN - 1) / kI4BN;
    const int tiles_m = (M + kI4BM - 1) / kI4BM;
    hipLaunchKernelGGL(w4a4_int4_kernel<W4Epilogue::kLinear>, dim3(tiles_n * tiles_m), dim3(kI4Threads), 0,
                       stream, qx, sx, T, qw, sw, l2t, bias, M, N, K, rank, Y, y_f32, nullptr, tiles_n);
    return hipGetLastError();
}

hipError_t launch_w4a4_partials(const uint8_t *qx, const uint8_t *qw, int M, int N, int K,
                                int32_t *P, hipStream_t stream) {
    const int tiles_n = (N + kI4BN - 1) / kI4BN;
    const int tiles_m = (M + kI4BM - 1) / kI4BM;
    hipLaunchKernelGGL(w4a4_int4_kernel<W4Epilogue::kPartials>, dim3(tiles_n * tiles_m), dim3(kI4Threads), 0,
                       stream, qx, nullptr, nullptr, qw, nullptr, nullptr, nullptr, M, N, K, 0, nullptr, false, P,
                       tiles_n);
    return hipGetLastError();
}

}  // namespace svdq
