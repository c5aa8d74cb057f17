// The MXFP4 variant of the SVDQuant W4A4 linear: FP4 E2M1 codes with E8M0
// scales per block of 32 along K (OCP microscaling) on gfx950's scaled MFMA,
// fused low-rank up-projection and bias.
//
// Source: "Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru),
// "Nunchaku Lite" paragraph (svdq_w4a4 in an INT4 and a 4-bit float variant)
// and method paragraph (4-bit weights x 4-bit activations with a 16-bit
// low-rank branch). The 4-bit float format here is MXFP4, gfx950's native
// one.
//
//   acc[n, m] = sum_b 2^(uw[b, n] + ux[b, m]) sum_{k in b} e2m1(qw) e2m1(qx)
//   y = acc + T L2 + bias  ->  bf16 (nearest even) or fp32
//
// One v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP4 covers two
// 32-blocks (a lane's 32 codes are one block, its scale byte that block's
// E8M0) and accumulates straight into the fp32 tile: the block scales are
// applied by the matrix core, so unlike the INT4 variant there is no
// per-group rescale on the vector ALU.
//
// Block tile 128 (n) x 128 (m), 4 waves as 2 x 2, wave tile 64 x 64 (2 x 2
// MFMA tiles of 32 x 32). One LDS stage holds two groups of 64 k: per
// operand the two groups' [2 halves][rows][16 bytes] tiles exactly as the MX
// container stores them (rows in blocks of 128, the halves of a group
// k-block-major, so 16 consecutive rows' 16-byte pieces are contiguous and
// an MFMA operand read touches every LDS bank once), plus the groups' E8M0
// bytes. Everything goes straight from global memory to LDS (buffer_load ...
// lds), 1 KB per operand load and 256 bytes per scale load. Three stages
// rotate: while one is read, the next two are in flight (a stage holds only
// eight MFMAs per wave, far less than a load's latency), with one barrier
// per stage. In a block with fewer than 128 rows
// the copy runs on into the next tile or past the end of the buffer (zeros);
// those rows feed only outputs that are never stored.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace svdq {

namespace {

constexpr int MX_BN = 128;
constexpr int MX_BM = 128;
constexpr int MX_THREADS = 256;
constexpr int MX_KG = 2;             // groups of 64 k per LDS stage
constexpr int MX_NS = 3;             // LDS stages: two in flight while one is read
constexpr int MX_TILE = 128 * 32;    // one group of a 128-row block: 4 KB
constexpr int MX_FP4 = 4;            // MFMA operand format: FP4 E2M1

typedef int32_t mx_i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void mx_lds_void;

struct StageMx {
    uint8_t a[MX_KG * MX_TILE];   // weights: [group][half][row][16 bytes]
    uint8_t b[MX_KG * MX_TILE];   // activations
    uint8_t ua[MX_KG][2][MX_BN];  // E8M0 of the weights: [group][half][row]
    uint8_t ub[MX_KG][2][MX_BM];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mx_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ mx_i32x8 frag4(const uint8_t *p) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(p);
    return mx_i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], 0, 0, 0, 0};
}

__global__ __launch_bounds__(MX_THREADS, 3) void mx_linear_kernel(
    const uint8_t *__restrict__ qx, const uint8_t *__restrict__ ux, const uint16_t *__restrict__ T,
    const uint8_t *__restrict__ qw, const uint8_t *__restrict__ uw, const uint16_t *__restrict__ l2t,
    const uint16_t *__restrict__ bias, int M, int N, int K, int ldm, int ldn, int rank,
    void *__restrict__ Y, bool y_f32, int tiles_n) {
    // the stages in separate LDS variables: the compiler can then tell a
    // stage being refilled (direct-to-LDS loads) from the one being read and
    // does not make the reads wait for the loads
    __shared__ __attribute__((aligned(16))) StageMx sm0;
    __shared__ __attribute__((aligned(16))) StageMx sm1;
    __shared__ __attribute__((aligned(16))) StageMx sm2;
    __shared__ __attribute__((aligned(16))) float bias_s[128];

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int n0 = tile_n * MX_BN;
    const int m0 = tile_m * MX_BM;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int G = K / 64;
    const int S = (G + MX_KG - 1) / MX_KG;
    const uint32_t R = (uint32_t)K / 2;
    const int nbA = min(128, N - n0);  // rows of this block in the weight container
    const int nbB = min(128, M - m0);

    const __amdgpu_buffer_rsrc_t rw = mx_rsrc(qw, (uint32_t)N * R);
    const __amdgpu_buffer_rsrc_t rx = mx_rsrc(qx, (uint32_t)M * R);
    const __amdgpu_buffer_rsrc_t ruw = mx_rsrc(uw, (uint32_t)(K / 32) * (uint32_t)ldn);
    const __amdgpu_buffer_rsrc_t rux = mx_rsrc(ux, (uint32_t)(K / 32) * (uint32_t)ldm);

    // Per stage the block issues 16 operand loads (per operand and group one
    // 4 KB tile, four 1 KB loads) and 4 scale loads; wave w takes operand
    // w / 2 and group w % 2 of the stage for both.
    const int op_w = wave >> 1, q_w = wave & 1;
    const uint32_t base_w = (uint32_t)(op_w ? m0 : n0) * R;
    const uint32_t tstride_w = (uint32_t)(op_w ? nbB : nbA) * 32u;  // bytes per group in the block
    // scale bytes: lanes 0-31 read half 0 (k-block 2g), lanes 32-63 half 1,
    // 4 rows per lane; the scale rows are ld bytes apart (ld % 16 == 0)
    const uint32_t ld_w = (uint32_t)(op_w ? ldm : ldn);
    const uint32_t soff_w = (uint32_t)lh * ld_w + (uint32_t)(op_w ? m0 : n0) + 4u * (uint32_t)r32;

    auto issue_stage = [&](int s, StageMx &st) {
        const int g = s * MX_KG + q_w;
        if (g < G) {
            const uint32_t t0 = base_w + (uint32_t)g * tstride_w + (uint32_t)lane * 16u;
            uint8_t *dst = (op_w ? st.b : st.a) + q_w * MX_TILE;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(op_w ? rx : rw, (mx_lds_void *)(dst + i * 1024), 16,
                                                         t0 + i * 1024, 0, 0, 0);
            uint8_t *sdst = op_w ? &st.ub[q_w][0][0] : &st.ua[q_w][0][0];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(op_w ? rux : ruw, (mx_lds_void *)sdst, 4,
                                                     soff_w + (uint32_t)(2 * g) * ld_w, 0, 0, 0);
        }
    };

    // this lane's operand byte offsets within a staged group tile: the
    // container's halves are nb * 16 bytes apart in a block of nb rows
    int aoff[2], boff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        aoff[i] = lh * nbA * 16 + (wn * 64 + i * 32 + r32) * 16;
        boff[i] = lh * nbB * 16 + (wm * 64 + i * 32 + r32) * 16;
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // loads this wave issues for stage t (operand tile + scales, or none
    // past K): the explicit waits below count them
    auto loads_of = [&](int t) { return (t < S && t * MX_KG + q_w < G) ? 5 : 0; };
    // wait until at most `pending` of this wave's loads are outstanding
    // (0 or 5: vmcnt is an immediate)
    auto wait_loads = [&](int pending) {
        __builtin_amdgcn_sched_barrier(0);
        if (pending)
            __builtin_amdgcn_s_waitcnt(5 | (7 << 4) | (0 << 8));  // vmcnt(5) lgkmcnt(0)
        else
            __builtin_amdgcn_s_waitcnt(0);
    };

    stage_bias_128(bias_s, bias, n0, N, tid);
    issue_stage(0, sm0);
    if (S > 1) issue_stage(1, sm1);
    wait_loads(loads_of(1));
    __syncthreads();

    // stage s is read from `cur` while stage s + 2 loads into `refill`
    auto run_stage = [&](int s, const StageMx &cur, StageMx &refill) {
        if (s + 2 < S) issue_stage(s + 2, refill);
        const int ng = min(MX_KG, G - s * MX_KG);
        mx_i32x8 a[MX_KG][2], b[MX_KG][2];
        int sa[MX_KG][2], sb[MX_KG][2];
#pragma unroll
        for (int q = 0; q < MX_KG; ++q) {
            if (q >= ng) break;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[q][i] = frag4(cur.a + q * MX_TILE + aoff[i]);
                b[q][i] = frag4(cur.b + q * MX_TILE + boff[i]);
                sa[q][i] = cur.ua[q][lh][wn * 64 + i * 32 + r32];
                sb[q][i] = cur.ub[q][lh][wm * 64 + i * 32 + r32];
            }
        }
        // the stage's MFMAs at raised wave priority, so that waves ready for
        // the matrix core issue before others' loads and LDS reads (measured
        // 5 % faster)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int q = 0; q < MX_KG; ++q) {
            if (q >= ng) break;
#pragma unroll
            for (int in = 0; in < 2; ++in)
#pragma unroll
                for (int im = 0; im < 2; ++im)
                    acc[in][im] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a[q][in], b[q][im], acc[in][im], MX_FP4, MX_FP4, 0, sa[q][in], 0, sb[q][im]);
        }
        __builtin_amdgcn_s_setprio(0);
        // stage s + 1 must have landed before anyone reads it (stage s + 2
        // may stay in flight), and everyone must be done with stage s before
        // it is refilled (with stage s + 3, issued after the barrier)
        wait_loads(loads_of(s + 2));
        __syncthreads();
    };
    // stage s lives in sm(s % 3)
    for (int s = 0; s < S; s += MX_NS) {
        run_stage(s, sm0, sm2);
        if (s + 1 < S) run_stage(s + 1, sm1, sm0);
        if (s + 2 < S) run_stage(s + 2, sm2, sm1);
    }

    // low-rank up-projection T L2 (bf16 MFMA, fp32 accumulation) and bias
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
    // every load has landed and been read: the stage buffers hold the
    // output tile on its way out
    static_assert(sizeof(StageMx) >= kTileHalfLdsBytes, "LDS too small for the output tile");
    store_tile_128x128(acc, reinterpret_cast<uint8_t *>(&sm0), reinterpret_cast<uint8_t *>(&sm1), bias_s, Y, y_f32, M,
                       N, m0, n0, wn, wm, tid);
}

}  // namespace

hipError_t launch_mx_linear(const uint8_t *qx, const uint8_t *ux, const uint16_t *T, const uint8_t *qw,
                            const uint8_t *uw, const uint16_t *l2t, const uint16_t *bias, int M, int N, int K,
                            int rank, void *Y, bool y_f32, hipStream_t stream) {
    const int tiles_n = (N + MX_BN - 1) / MX_BN;
    const int tiles_m = (M + MX_BM - 1) / MX_BM;
    hipLaunchKernelGGL(mx_linear_kernel, dim3(tiles_n * tiles_m), dim3(MX_THREADS), 0, stream, qx, ux, T, qw, uw,
                       l2t, bias, M, N, K, (int)mx_scale_ld(M), (int)mx_scale_ld(N), rank, Y, y_f32, tiles_n);
    return hipGetLastError();
}

}  // namespace svdq
