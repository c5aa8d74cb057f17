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
// and no integer-to-float conversion. The scale products sx[g, m] sw[g, n]
// come from the matrix core too: an fp32 MFMA with K = 1 is an outer
// product, and the two-block v_mfma_f32_32x32x1_2b_f32 returns the products
// of two 32 x 32 tiles in the same lane layout as their partials, each
// rounded once as a VALU multiply rounds it. The vector ALU does one FMA per
// output element and group.
//
// Block tile 128 (n) x 128 (m), 4 waves as 2 x 2, wave tile 64 x 64 (2 x 2
// MFMA tiles of 32 x 32); for shapes whose 128 x 128 tiles would leave a
// last round of block slots mostly empty, 128 x 64 (wave tile 64 x 32, four
// blocks per CU; the plain store epilogue only). One LDS stage holds two
// groups (K = 128): per operand the two groups' [128 rows][48 bytes] tiles
// (64 token rows in the 128 x 64 tile), exactly as the FP6
// container stores them (rows in blocks of 128, each block's groups one after
// another), plus the two groups' 2 x 128 scales. Operands and scales go
// straight from global memory to LDS (buffer_load ... lds, 16 or 4 bytes per
// lane, lane l to base + l * size): no registers, no LDS store instructions.
// A stage's operand tile is 6 KB of contiguous memory, copied 1 KB per load,
// so every load is fully coalesced. Rows are 48 bytes apart, which already
// spreads the 16-byte operand reads of 16 consecutive rows over all LDS
// banks. In a block holding fewer than 128 rows (the tail of M or N) the
// load runs on into the next tile or past the end of the buffer, where it
// reads zeros (the whole offset is in the per-lane offset, so the range
// check sees it); the extra rows only feed outputs that are never stored. A
// lane half's 24-byte MFMA operand is one 16-byte read of its plane and one
// 8-byte read of the shared third plane. Stages are double buffered with one
// barrier per stage; the next stage's loads are in flight during the current
// stage's MFMAs.
//
// The MLP epilogue (an up-projection feeding a down-projection through GELU)
// does not store y: it rounds y to bf16, applies GELU and quantizes the
// result for the down-projection in place -- per token row and group of 64
// output columns the INT4 codes (FP6 container) and the fp32 group scale,
// and the tile's share of the down-projection's low-rank T.

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "gelu.h"
#include "internal.h"
#include "quant_common.h"

namespace svdq {

namespace {

constexpr int BN = 128;
constexpr int BM = 128;
constexpr int THREADS = 256;
constexpr int KG = 2;            // groups per LDS stage
constexpr int GB = 48;           // container bytes per row and group
constexpr int E8M0_X8 = 127 + 3; // MFMA block scale 2^3

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int TILE = 128 * GB;  // one group of a 128-row block: 6 KB

// what the kernel does after the main loop
constexpr int kEpiStore = 0;     // y = acc + T L2 + bias, stored (svdq_w4a4_linear)
constexpr int kEpiPartials = 1;  // int32 group partials stored per group (debug entry point)
constexpr int kEpiMlp = 2;       // y -> bf16 -> GELU -> the down-projection's activation side

// one LDS stage of a block with kRowsB token rows (128, or 64 in the
// 64-row tile variant)
template <int kRowsB>
struct Stage6T {
    uint8_t a[KG * TILE];           // [group][row][48 bytes]
    uint8_t b[KG * kRowsB * GB];
    float sa[KG][BN];
    float sb[KG][kRowsB];
};
using Stage6 = Stage6T<BM>;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// the 24-byte MFMA operand from a staged region; off16/off8 are the byte
// offsets (within the region) of the lane's 16-byte and 8-byte pieces
__device__ __forceinline__ i32x8 frag6(const uint8_t *region, int off16, int off8) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(region + off16);
    const u32x2 y = *reinterpret_cast<const u32x2 *>(region + off8);
    return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], 0, 0};
}

// LDS of the MLP epilogue (the stage buffers are free by then): in the
// first stage buffer a bf16 tile of 64 rows x 128 columns (rows padded to
// 264 bytes), 1 / s and s of the tile's 128 channels, and the GELU table;
// in the second the tile's other 64 rows at the same pitch.
constexpr int kMlpPitch = 264;
constexpr int kMlpRcpOff = 64 * kMlpPitch;
constexpr int kMlpSOff = kMlpRcpOff + 128 * 8;
constexpr int kMlpTabOff = kMlpSOff + 128 * 4;
constexpr int kMlpLdsBytes = kMlpTabOff + kGeluTableEntries * 2;

// The tile's y = acc + bias, rounded to bf16, goes into LDS whole (rows
// 0..63 in lds, 64..127 in lds_hi), so the accumulators are dead before the
// quantizer runs. Then in two passes of 64 token rows, thread t takes row
// t / 4 and the 32 channels 32 (t % 4) of it:
// (optionally) stores y_up, replaces y by g = GELU(y) in the tile, and
// quantizes g as the standalone activation pass does: x_hat = fp32(g / s)
// (computed once, held in registers), the group absmax over its 32
// channels and the partner thread's (t ^ 1,
// the other half of the group), scale = absmax / 7, codes by nearest even,
// written as FP6 fields straight into the down-projection's container (the
// tile's rows are one 128-row block of it, its 128 columns two groups).
// Last, wave w multiplies rows 16 w .. 16 w + 15 of the g tile by the
// tile's 128 rows of L1s (16x16x32 bf16 MFMAs, fp32 accumulation) and
// stores the fp32 partial of T for this column tile. Columns past N (N is
// a multiple of 64, so a whole group) give g = 0 and are not written.
__device__ __forceinline__ void mlp_epilogue(const f32x16 (&acc)[2][2], uint8_t *lds, uint8_t *lds_hi,
                                             const float *bias_s,
                                             const MlpOut &o, int M, int N,
                                             int m0, int n0, int tile_n, int wn, int wm, int tid) {
    const int lane = tid & 63, r32 = lane & 31, lh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    double *rcp = reinterpret_cast<double *>(lds + kMlpRcpOff);
    float *sv = reinterpret_cast<float *>(lds + kMlpSOff);
    uint16_t *tab = reinterpret_cast<uint16_t *>(lds + kMlpTabOff);
    if (tid < 128) {
        const float sg = n0 + tid < N ? o.smooth[n0 + tid] : 1.0f;
        sv[tid] = sg;
        rcp[tid] = 1.0 / (double)sg;
    }
    for (int i = tid; i < kGeluTableEntries / 8; i += THREADS)
        reinterpret_cast<u32x4 *>(tab)[i] = reinterpret_cast<const u32x4 *>(kGeluTable)[i];

    const int row = tid >> 2, qd = tid & 3, gl = qd >> 1, half = qd & 1;
    const bool grp_ok = n0 + 64 * gl < N;
    const int nb = min(128, M - m0);  // rows of this block of the container
    const int g_down = 2 * (n0 / 128) + gl;
    // the whole y tile into LDS first (rows 0..63 in lds, 64..127 in
    // lds_hi), so that the accumulators are dead before the quantizer runs
#pragma unroll
    for (int in = 0; in < 2; ++in) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int nl = wn * 64 + in * 32 + 8 * qq + 4 * lh;
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(bias_s + nl);
#pragma unroll
            for (int im = 0; im < 2; ++im) {
                const int ml = im * 32 + r32;
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = acc[in][im][4 * qq + t] + bv[t];
                *reinterpret_cast<u32x2 *>((wm ? lds_hi : lds) + ml * kMlpPitch + nl * 2) =
                    u32x2{bf16x2_bits(v[0], v[1]), bf16x2_bits(v[2], v[3])};
            }
        }
    }
    __syncthreads();
    for (int p = 0; p < 2; ++p) {
        uint8_t *tile = p ? lds_hi : lds;
        const int m = m0 + 64 * p + row;
        uint8_t *rowp = tile + row * kMlpPitch + 64 * qd;
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x2 x = reinterpret_cast<const u32x2 *>(rowp)[i];
            w[2 * i] = x[0];
            w[2 * i + 1] = x[1];
        }
        if (o.y_up && grp_ok && m < M) {
            uint16_t *dst = o.y_up + (size_t)m * N + n0 + 32 * qd;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                reinterpret_cast<u32x4 *>(dst)[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        }
        // g = GELU(y), back into the tile (zero past N)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t lo = gelu_bf16_bits(w[i] & 0xFFFFu, tab);
            const uint32_t hi = gelu_bf16_bits(w[i] >> 16, tab);
            w[i] = grp_ok ? (lo | (hi << 16)) : 0u;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) reinterpret_cast<u32x2 *>(rowp)[i] = u32x2{w[2 * i], w[2 * i + 1]};

        // x_hat = fp32(g / s): exact through fp64 reciprocals (quotient_fp32),
        // computed once (g and 1 / s read back from LDS eight channels at a
        // time) and held for the codes: the main loop's registers are free
        // by now
        auto chunk = [&](int c, float gv[8]) {
            // rows are 8-byte aligned (264-byte pitch): two 8-byte reads
            const u32x2 x0 = reinterpret_cast<const u32x2 *>(rowp)[2 * c];
            const u32x2 x1 = reinterpret_cast<const u32x2 *>(rowp)[2 * c + 1];
            const uint32_t x[4] = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gv[2 * i] = bf16_bits_to_f32(x[i] & 0xFFFFu);
                gv[2 * i + 1] = bf16_bits_to_f32(x[i] >> 16);
            }
        };
        float amax = 0.0f;
        float xq[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float gv[8];
            chunk(c, gv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                xq[8 * c + i] = quotient_fp32(gv[i], rcp[32 * qd + 8 * c + i]);
                amax = fmaxf(amax, fabsf(xq[8 * c + i]));
            }
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        // below the range quotient_fp32 covers: IEEE divisions (both threads
        // of the group decide alike)
        const bool tiny = amax < kTinyGroup;
        if (tiny) {
            amax = 0.0f;
#pragma unroll 1
            for (int c = 0; c < 4; ++c) {
                float gv[8];
                chunk(c, gv);
#pragma unroll
                for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(gv[i] / sv[32 * qd + 8 * c + i]));
            }
            amax = fmaxf(amax, __shfl_xor(amax, 1));
        }
        // fp32(amax / 7): amax is 0 or at least 2^-100 unless the group is
        // tiny, where the IEEE division is kept
        const float scale = tiny ? amax / 7.0f : quotient_fp32(amax, kRcp7);
        const double rscale = scale != 0.0f ? 1.0 / (double)scale : 0.0;
        // 32 six-bit fields, LSB first, 16 codes (two chunks) per packing
        // conversion: codes 16 hh .. 16 hh + 15 fill fw[3 hh .. 3 hh + 2]
        uint32_t fw[6] = {0u, 0u, 0u, 0u, 0u, 0u};
        if (scale != 0.0f) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float v[16];
                if (tiny) {
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const int c = 2 * hh + cc;
                        float gv[8];
                        chunk(c, gv);
#pragma unroll
                        for (int i = 0; i < 8; ++i) v[8 * cc + i] = fp6_value(gv[i] / sv[32 * qd + 8 * c + i], rscale);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) v[i] = fp6_value(xq[16 * hh + i], rscale);
                }
                uint32_t w3[3];
                pack_fp6_16(v, w3);
                fw[3 * hh] = w3[0];
                fw[3 * hh + 1] = w3[1];
                fw[3 * hh + 2] = w3[2];
            }
        }
        if (grp_ok && m < M) {
            // the row's 48 bytes of group g_down: this half's 24 bytes H as
            // H[0:16] at 16 half and H[16:24] at 32 + 8 half
            uint8_t *rec = o.qx + (size_t)m0 * (size_t)(N / 4 * 3) + ((size_t)g_down * nb + (m - m0)) * GB;
            *reinterpret_cast<u32x4 *>(rec + 16 * half) = u32x4{fw[0], fw[1], fw[2], fw[3]};
            *reinterpret_cast<u32x2 *>(rec + 32 + 8 * half) = u32x2{fw[4], fw[5]};
            if (half == 0) o.sx[(size_t)g_down * M + m] = scale;
        }
        __syncthreads();

        // this pass's share of T: rows 16 wave + (lane % 16), channels
        // 32 step + 8 (lane / 16) + i of the tile
        if (o.rank > 0) {
            f32x4 tacc[SVDQ_MAX_RANK / 16];
#pragma unroll
            for (int rt = 0; rt < SVDQ_MAX_RANK / 16; ++rt) tacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int ar = 16 * wave + (lane & 15);
#pragma unroll
            for (int step = 0; step < 4; ++step) {
                const int kc = 32 * step + 8 * (lane >> 4);
                const uint8_t *ap = tile + ar * kMlpPitch + kc * 2;
                const u32x2 a0 = reinterpret_cast<const u32x2 *>(ap)[0];
                const u32x2 a1 = reinterpret_cast<const u32x2 *>(ap)[1];
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
                const bool k_ok = n0 + 32 * step < N;
#pragma unroll
                for (int rt = 0; rt < SVDQ_MAX_RANK / 16; ++rt) {
                    if (rt * 16 < o.rank) {
                        u32x4 bw = {0u, 0u, 0u, 0u};
                        if (k_ok)
                            bw = *reinterpret_cast<const u32x4 *>(o.l1t + (size_t)(rt * 16 + (lane & 15)) * N + n0 + kc);
                        tacc[rt] = mfma_bf16_16x16x32(a, __builtin_bit_cast(bf16x8, bw), tacc[rt]);
                    }
                }
            }
            // 16x16 output: lane holds column (lane % 16) = rank index within
            // the tile, rows 4 (lane / 16) + t
#pragma unroll
            for (int rt = 0; rt < SVDQ_MAX_RANK / 16; ++rt) {
                if (rt * 16 < o.rank) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int mt = m0 + 64 * p + 16 * wave + 4 * (lane >> 4) + t;
                        if (mt < M)
                            o.tpart[((size_t)tile_n * M + mt) * o.rank + rt * 16 + (lane & 15)] = tacc[rt][t];
                    }
                }
            }
        }
        __syncthreads();
    }
}

// kBMt = 128, or 64 (a 128 x 64 block tile, plain store epilogue only: the
// same per-wave work for one 32-token slice instead of two, at four blocks
// per CU instead of three, for shapes whose 128 x 128 tiles leave most
// block slots of a last round empty)
template <int kEpi, int kBMt = BM>
__global__ __launch_bounds__(THREADS, kBMt == BM ? 3 : 4) void w4a4_fp6_kernel(
    const uint8_t *__restrict__ qx, const float *__restrict__ sx, const uint16_t *__restrict__ T,
    const uint8_t *__restrict__ qw, const float *__restrict__ sw, const uint16_t *__restrict__ l2t,
    const uint16_t *__restrict__ bias, int M, int N, int K, int rank, void *__restrict__ Y, bool y_f32,
    int32_t *__restrict__ Pout, int tiles_n, MlpOut mlp) {
    constexpr bool kLinear = kEpi != kEpiPartials;
    constexpr bool kHalf = kBMt != BM;
    static_assert(kBMt == BM || (kBMt == 64 && kEpi == kEpiStore), "64-row tiles: plain store epilogue only");
    constexpr int kTileB = kBMt * GB;    // one group of the block's token rows
    constexpr int kSlices = kBMt / 64;   // 32-token slices per wave
    // two stages in separate LDS variables: the compiler can then tell the
    // stage being refilled (direct-to-LDS loads) from the one being read and
    // does not make the reads wait for the loads
    __shared__ __attribute__((aligned(16))) Stage6T<kBMt> st0;
    __shared__ __attribute__((aligned(16))) Stage6T<kBMt> st1;

    const int tile_n = blockIdx.x % tiles_n;
    const int tile_m = blockIdx.x / tiles_n;
    const int n0 = tile_n * BN;
    const int m0 = tile_m * kBMt;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave & 1;
    const int wm = wave >> 1;
    const int mw0 = wm * 32 * kSlices;  // the wave's first token row in the block
    const int r32 = lane & 31;
    const int lh = lane >> 5;
    const int G = K / 64;
    const int S = (G + KG - 1) / KG;
    const uint32_t R = (uint32_t)K / 4 * 3;

    const __amdgpu_buffer_rsrc_t rw = make_rsrc(qw, (uint32_t)N * R);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(qx, (uint32_t)M * R);
    const __amdgpu_buffer_rsrc_t rsw = make_rsrc(sw, (uint32_t)G * (uint32_t)N * 4u);
    const __amdgpu_buffer_rsrc_t rsx = make_rsrc(sx, (uint32_t)G * (uint32_t)M * 4u);

    // Per stage the block issues 24 operand loads (per operand and group one
    // 6 KB tile, six 1 KB loads; 3 KB, three loads, for 64 token rows); wave
    // w loads tile w (operand w / 2, group w % 2 of the stage). A 64-row
    // token tile is the first or second half of its 128-row container block:
    // each group's 64 rows are one contiguous 3 KB piece of the block's group
    // tile. The stage's scales of one side are two runs of 4 bytes per row
    // (one per group) in memory and one [2][rows] array in LDS: with four
    // rows per lane, one 16-byte load per side puts both runs in place
    // (wave 2 the weight side, wave 3 the token side). That needs the runs
    // to start on 16 bytes, i.e. a row count that is a multiple of 4 (N
    // always is; for M % 4 != 0 the token side takes one 4-byte load per
    // group and 64-row half, by waves 2 and 3). A lane's 16 bytes then lie
    // wholly inside or wholly past the end of the buffer.
    const int op_w = wave >> 1, q_w = wave & 1;
    const int rows_w = op_w ? M : N;
    const int b0_w = op_w ? (m0 & ~127) : n0;            // first row of the 128-row block
    const uint32_t base_w = (uint32_t)b0_w * R + (op_w ? (uint32_t)(m0 - b0_w) * GB : 0u);
    const uint32_t tstride_w = (uint32_t)min(128, rows_w - b0_w) * GB;  // bytes per group in the block
    const int nld_w = op_w ? kTileB / 1024 : TILE / 1024;  // 1 KB loads per group tile
    const bool sx16 = (M & 3) == 0;
    // the lane's scale piece: side (1: weights), its group within the stage
    // and its byte offset within that group's run
    const int s_side = wave == 2;
    const int s_per = s_side ? BN / 4 : kBMt / 4;  // lanes per group
    const bool s_lane = wave >= 2 && lane < 2 * s_per;
    const int s_slot = lane / s_per;
    const uint32_t s_off = (uint32_t)((s_side ? n0 : m0) + 4 * (lane % s_per)) * 4u;
    // byte offsets of this lane's operand pieces within a staged operand:
    // row r's 16-byte piece of plane lh at r * 48 + 16 lh, its 8-byte piece
    // of plane 2 at r * 48 + 32 + 8 lh; tile i (rows + 32 i) and slot q
    // (+ q TILE) are immediates. The 8-byte pieces of the two row tiles get
    // bases the compiler cannot see through: otherwise it pairs them into
    // one ds_read2 and needs moves to place each half next to its 16-byte
    // piece in the MFMA operand.
    const int a16 = (wn * 64 + r32) * GB + 16 * lh;
    const int b16 = (mw0 + r32) * GB + 16 * lh;
    int a8[2], b8[kSlices];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        a8[i] = (wn * 64 + i * 32 + r32) * GB + 32 + 8 * lh;
        asm volatile("" : "+v"(a8[i]));
    }
#pragma unroll
    for (int i = 0; i < kSlices; ++i) {
        b8[i] = (mw0 + i * 32 + r32) * GB + 32 + 8 * lh;
        asm volatile("" : "+v"(b8[i]));
    }

    // Every offset is carried whole in the per-lane offset, so a load that
    // runs past the end of its buffer is caught by the range check and
    // reads zeros. A group past K is never read and not loaded.
    auto issue_stage = [&](int s, Stage6T<kBMt> &st) {
        const int g = s * KG + q_w;
        if (g < G) {
            const uint32_t t0 = base_w + (uint32_t)g * tstride_w + (uint32_t)lane * 16u;
            uint8_t *dst = op_w ? st.b + q_w * kTileB : st.a + q_w * TILE;
#pragma unroll
            for (int i = 0; i < 6; ++i)
                if (i < nld_w)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(op_w ? rx : rw, (lds_void *)(dst + i * 1024), 16,
                                                             t0 + i * 1024, 0, 0, 0);
        }
        if constexpr (kLinear) {
            if (sx16 || s_side) {
                // a group past G lies past the end of the buffer: zeros, never read
                const uint32_t L = s_side ? (uint32_t)N : (uint32_t)M;
                if (s_lane)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(s_side ? rsw : rsx,
                                                             (lds_void *)(s_side ? &st.sa[0][0] : &st.sb[0][0]), 16,
                                                             (uint32_t)(s * KG + s_slot) * L * 4u + s_off, 0, 0, 0);
            }
            if (!sx16 && wave >= 2) {
                // token scales 4 bytes per lane: wave 2 group 0, wave 3 group
                // 1 of the stage, each in 64-row halves
                const int slot = wave - 2, gs = s * KG + slot;
#pragma unroll
                for (int half = 0; half < kBMt / 64; ++half)
                    if (gs < G)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            rsx, (lds_void *)(st.sb[slot] + half * 64), 4,
                            ((uint32_t)gs * (uint32_t)M + (uint32_t)(m0 + half * 64 + lane)) * 4u, 0, 0, 0);
            }
        }
    };

    f32x16 acc[2][kSlices];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kSlices; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const f32x32 zero32 = {};

    __shared__ __attribute__((aligned(16))) float bias_s[BN];
    if constexpr (kLinear) stage_bias_128(bias_s, bias, n0, N, tid);
    issue_stage(0, st0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // stage s is read from `cur` while stage s + 1 loads into `nxt`
    auto run_stage = [&](int s, const Stage6T<kBMt> &cur, Stage6T<kBMt> &nxt) {
        if (s + 1 < S) issue_stage(s + 1, nxt);
        const int ng = min(KG, G - s * KG);
#pragma unroll
        for (int q = 0; q < KG; ++q) {
            if (q >= ng) break;
            if constexpr (kLinear) {
                // per token slice im: one two-block fp32 MFMA (K = 1) gives
                // the scale products sw[n] sx[m] of tiles (0, im) and (1, im)
                // in the partials' layout (A = sw of the wave's 64 weight
                // rows, lane l: row l; B = sx of the slice's 32 tokens, lanes
                // l and l + 32: token l % 32), rounded once as a VALU multiply
                // would; the vector ALU is left one FMA per element
                const i32x8 a0 = frag6(cur.a, q * TILE + a16, q * TILE + a8[0]);
                const i32x8 a1 = frag6(cur.a, q * TILE + a16 + 32 * GB, q * TILE + a8[1]);
                const float swv = cur.sa[q][wn * 64 + lane];
#pragma unroll
                for (int im = 0; im < kSlices; ++im) {
                    // keep the scheduler from hoisting the next slice's
                    // operands (and their registers) into this one
                    __builtin_amdgcn_sched_barrier(0);
                    const i32x8 bm = frag6(cur.b, q * kTileB + b16 + im * 32 * GB, q * kTileB + b8[im]);
                    const float sxv = cur.sb[q][mw0 + im * 32 + r32];
                    // the slice's MFMAs are issued at raised wave priority
                    // and its FMAs at the normal one, so that waves ready
                    // for the matrix core go first (2 % faster in an earlier
                    // form of this loop; no measurable difference, either
                    // way, in this one)
                    __builtin_amdgcn_s_setprio(1);
                    const f32x32 C = __builtin_amdgcn_mfma_f32_32x32x1f32(swv, sxv, zero32, 0, 0, 0);
                    const f32x16 P0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bm, zero16, 2, 2, 0,
                                                                                      E8M0_X8, 0, E8M0_X8);
                    const f32x16 P1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bm, zero16, 2, 2, 0,
                                                                                      E8M0_X8, 0, E8M0_X8);
                    __builtin_amdgcn_s_setprio(0);
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[0][im][e] = fmaf(C[e], P0[e], acc[0][im][e]);
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[1][im][e] = fmaf(C[16 + e], P1[e], acc[1][im][e]);
                }
            } else {
                i32x8 a[2], b[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    a[i] = frag6(cur.a, q * TILE + a16 + i * 32 * GB, q * TILE + a8[i]);
                    b[i] = frag6(cur.b, q * TILE + b16 + i * 32 * GB, q * TILE + b8[i]);
                }
#pragma unroll
                for (int in = 0; in < 2; ++in) {
#pragma unroll
                    for (int im = 0; im < 2; ++im) {
                        const f32x16 P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            a[in], b[im], zero16, 2, 2, 0, E8M0_X8, 0, E8M0_X8);
                        const int g = s * KG + q;
                        const int m = m0 + wm * 64 + im * 32 + r32;
                        if (m < M) {
#pragma unroll
                            for (int qq = 0; qq < 4; ++qq) {
                                const int n = n0 + wn * 64 + in * 32 + 8 * qq + 4 * lh;
                                if (n < N) {
                                    i32x4 v;
#pragma unroll
                                    for (int u = 0; u < 4; ++u) v[u] = (int)P[4 * qq + u];
                                    *reinterpret_cast<i32x4 *>(Pout + ((size_t)g * M + m) * N + n) = v;
                                }
                            }
                        }
                    }
                }
            }
        }
        // the next stage's direct-to-LDS loads must have landed before anyone
        // reads them, and everyone must be done with this stage before it is
        // refilled
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    for (int s = 0; s < S; s += 2) {
        run_stage(s, st0, st1);
        if (s + 1 < S) run_stage(s + 1, st1, st0);
    }

    if constexpr (kLinear) {
        for (int kk = 0; kk < rank; kk += 16) {
            bf16x8 la[2], lb[kSlices];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int n = n0 + wn * 64 + i * 32 + r32;
                u32x4 va = {0u, 0u, 0u, 0u};
                if (n < N) va = *reinterpret_cast<const u32x4 *>(l2t + (size_t)n * rank + kk + 8 * lh);
                la[i] = __builtin_bit_cast(bf16x8, va);
            }
#pragma unroll
            for (int i = 0; i < kSlices; ++i) {
                const int m = m0 + mw0 + i * 32 + r32;
                u32x4 vb = {0u, 0u, 0u, 0u};
                if (m < M) vb = *reinterpret_cast<const u32x4 *>(T + (size_t)m * rank + kk + 8 * lh);
                lb[i] = __builtin_bit_cast(bf16x8, vb);
            }
#pragma unroll
            for (int in = 0; in < 2; ++in)
#pragma unroll
                for (int im = 0; im < kSlices; ++im) acc[in][im] = mfma_bf16_32x32x16(la[in], lb[im], acc[in][im]);
        }
        // every load has landed and been read: the stage buffers hold the
        // output tile on its way out
        if constexpr (kHalf) {
            static_assert(sizeof(Stage6T<kBMt>) >= kTile64LdsBytes, "LDS too small for the output tile");
            store_tile_128x64(acc, reinterpret_cast<uint8_t *>(&st0), bias_s, Y, y_f32, M, N, m0, n0, wn, wm, tid);
        } else {
            static_assert(sizeof(Stage6) >= kTileHalfLdsBytes, "LDS too small for the output tile");
            static_assert(sizeof(Stage6) >= kMlpLdsBytes, "LDS too small for the MLP epilogue");
            if constexpr (kEpi == kEpiMlp)
                mlp_epilogue(acc, reinterpret_cast<uint8_t *>(&st0), reinterpret_cast<uint8_t *>(&st1), bias_s, mlp, M,
                             N, m0, n0, tile_n, wn, wm, tid);
            else
                store_tile_128x128(acc, reinterpret_cast<uint8_t *>(&st0), reinterpret_cast<uint8_t *>(&st1),
                                   bias_s, Y, y_f32, M, N, m0, n0, wn, wm, tid);
        }
    }
}

}  // namespace

static bool fp6_use_64_row_tiles(int M, int N) {
    // The kernel is bound by its per-SIMD MFMA and VALU work, so a CU's time
    // follows the tile work it is dealt: 128 x 128 tiles at three blocks per
    // CU, or 128 x 64 tiles (half the work each) at four. Dealt round-robin
    // over kCUs CUs, the busiest CU gets ceil(tiles / kCUs) tiles; the
    // 64-row tiles are used when that is at least 10 % less work, and when
    // the 128 x 128 tiles are too few to give every CU one (a CU with a
    // single block of four waves waits on latency; measured 24 % faster with
    // the 64-row tiles at 1024 x 3072 x 3072). Measured over nine shapes
    // (1024-32760 tokens, N 3072-12288), this picks the faster tiling in each.
    constexpr int64_t kCUs = 256;  // MI355X
    const int64_t tn = (N + BN - 1) / BN;
    const int64_t tiles = tn * ((M + BM - 1) / BM);                      // 128 x 128 tiles
    const int64_t full = (tiles + kCUs - 1) / kCUs;
    const int64_t half = (tn * ((M + 63) / 64) + kCUs - 1) / kCUs;     // 128 x 64 tiles
    return tiles <= kCUs || 10 * half < 9 * 2 * full;
}

hipError_t launch_w4a4_fp6_linear(const uint8_t *qx, const float *sx, const uint16_t *T, const uint8_t *qw,
                                  const float *sw, const uint16_t *l2t, const uint16_t *bias, int M, int N,
                                  int K, int rank, void *Y, bool y_f32, hipStream_t stream) {
    const int tiles_n = (N + BN - 1) / BN;
    if (fp6_use_64_row_tiles(M, N)) {
        const int tiles_m = (M + 63) / 64;
        hipLaunchKernelGGL((w4a4_fp6_kernel<kEpiStore, 64>), dim3(tiles_n * tiles_m), dim3(THREADS), 0, stream, qx,
                           sx, T, qw, sw, l2t, bias, M, N, K, rank, Y, y_f32, nullptr, tiles_n, MlpOut{});
        return hipGetLastError();
    }
    const int tiles_m = (M + BM - 1) / BM;
    hipLaunchKernelGGL(w4a4_fp6_kernel<kEpiStore>, dim3(tiles_n * tiles_m), dim3(THREADS), 0, stream, qx, sx, T,
                       qw, sw, l2t, bias, M, N, K, rank, Y, y_f32, nullptr, tiles_n, MlpOut{});
    return hipGetLastError();
}

int mlp_tiles_n(int N) { return (N + BN - 1) / BN; }

hipError_t launch_w4a4_fp6_mlp(const uint8_t *qx, const float *sx, const uint16_t *T, const uint8_t *qw,
                               const float *sw, const uint16_t *l2t, const uint16_t *bias, int M, int N, int K,
                               int rank, const MlpOut &out, hipStream_t stream) {
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles_m = (M + BM - 1) / BM;
    hipLaunchKernelGGL(w4a4_fp6_kernel<kEpiMlp>, dim3(tiles_n * tiles_m), dim3(THREADS), 0, stream, qx, sx, T,
                       qw, sw, l2t, bias, M, N, K, rank, nullptr, false, nullptr, tiles_n, out);
    return hipGetLastError();
}

hipError_t launch_w4a4_fp6_partials(const uint8_t *qx, const uint8_t *qw, int M, int N, int K, int32_t *P,
                                    hipStream_t stream) {
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles_m = (M + BM - 1) / BM;
    hipLaunchKernelGGL(w4a4_fp6_kernel<kEpiPartials>, dim3(tiles_n * tiles_m), dim3(THREADS), 0, stream, qx,
                       nullptr, nullptr, qw, nullptr, nullptr, nullptr, M, N, K, 0, nullptr, false, P, tiles_n,
                       MlpOut{});
    return hipGetLastError();
}

}  // namespace svdq
