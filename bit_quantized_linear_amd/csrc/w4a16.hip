// W4A16 linear -- the awq_w4a16 layer type: INT4 group-64 weights, bf16
// activations ("Hugging Face встроила Nunchaku в Diffusers..." (iitog.ru),
// "Nunchaku Lite" paragraph: 4-bit weights with 16-bit activations for the
// precision-sensitive normalization and modulation layers).
//
// Those layers take the conditioning vector of each sample, so M is a batch
// of a few rows and the layer is a skinny GEMM whose cost is reading the
// packed weight once: HBM-bound. Each block owns 32 output columns and at
// most 16 batch rows; its waves split K. The weight container is streamed in
// 2304-byte units (32 columns x 128 k of codes plus their 64 scales), three
// 16-byte loads per lane and unit, several units in flight per wave. The
// block's rows of X are copied into LDS once (direct-to-LDS loads), so the
// MFMA A fragments cost LDS reads instead of vector-memory address work,
// which is what limits a skinny kernel that loads its activations per unit.
// The arithmetic runs on bf16 MFMA (16x16x32) with the batch padded to 16.
//
// Exact decode without a subtraction: a nibble u = q + 8 OR-ed into the bf16
// pattern 0x4300 is the bf16 number 128 + u = 136 + q, two codes per 32-bit
// AND-OR. A group's MFMA therefore gives sum_k x_k (136 + q_k); the bias
// 136 * sum_k x_k is removed by starting the accumulation at
// sum_k x_k (-136), an MFMA of the same A against a B operand of -136.
// Every product x (136 + q) and x 136 is exact in fp32; the cancellation
// costs a few fp32 ulps of 136 sum |x|, far below the bf16 rounding of y.

#include "device_common.h"
#include "internal.h"

namespace svdq {

namespace {

constexpr int kW16Depth = 4;               // units in flight per wave
constexpr int kW16Unit = 2304;             // 2 x 1024 B codes + 256 B scales
constexpr int kW16Rows = 16;               // batch rows per block at most (MFMA M)
constexpr uint32_t kW16LdsMax = 56u << 10;  // dynamic LDS of a block: its rows of X

typedef __attribute__((address_space(3))) void w16_lds_void;

// One unit in registers: the lane's 16 code bytes of each of the NT tiles
// the block computes, and the 4 scales of column lane % 16: (tile 0,
// tile 1) x (group 2p, 2p + 1).
template <int NT>
struct W16Unit {
    u32x4 code[NT];
    u32x4 scale;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t w16_rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// (w & mask) | magic as one v_and_or_b32. Its encoding takes neither
// literal constants nor two scalar operands, so the mask comes in as a
// kernel argument (an SGPR) and the magic as a VGPR copied once at the
// start of the kernel (a plain move, before any MFMA is issued).
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask_s, uint32_t magic_v) {
    return (w & mask_s) | magic_v;
}

// 8 nibbles (u = q + 8; codes j = 2i at bits 4i, j = 2i + 1 at bits 16 + 4i)
// -> 8 bf16 values 136 + q_j in k order: 4 AND-ORs and 3 shifts.
__device__ __forceinline__ bf16x8 w16_decode(uint32_t w, uint32_t mask_s, uint32_t magic_v) {
    u32x4 v;
    v[0] = and_or(w, mask_s, magic_v);
    v[1] = and_or(w >> 4, mask_s, magic_v);
    v[2] = and_or(w >> 8, mask_s, magic_v);
    v[3] = and_or(w >> 12, mask_s, magic_v);
    return __builtin_bit_cast(bf16x8, v);
}

// Loads of one unit: codes and scales through buffer loads whose per-lane
// offsets are fixed (the unit offset rides in soffset) ...
template <int NT>
__device__ __forceinline__ void w16_load_w(W16Unit<NT> &r, __amdgpu_buffer_rsrc_t rw, uint32_t unit,
                                           uint32_t code_off, uint32_t scale_off) {
#pragma unroll
    for (int j = 0; j < NT; ++j)
        r.code[j] = __builtin_bit_cast(u32x4,
                                       __builtin_amdgcn_raw_buffer_load_b128(rw, code_off + 1024u * j, unit, 0));
    r.scale = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, scale_off, unit, 0));
}

// ... and its four A fragments from the LDS copy of X: group e's two 32-k
// steps at byte offsets xoff[e] and xoff[e] + 64.
__device__ __forceinline__ void w16_load_x(u32x4 x[4], const uint8_t *xs, const uint32_t xoff[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        x[2 * e] = *reinterpret_cast<const u32x4 *>(xs + xoff[e]);
        x[2 * e + 1] = *reinterpret_cast<const u32x4 *>(xs + xoff[e] + 64);
    }
}

// acc[j] += sw[j, g] * (sum_{k in g} x (136 + q) - 136 sum_{k in g} x) for
// the two groups g of the unit and its NT tiles j (tile j0 + j of the
// unit): the -136 S term comes from MFMAs against a B operand of -136
// (x * 136 is exact in fp32) and seeds the tiles' accumulations.
template <int NT>
__device__ __forceinline__ void w16_compute(const W16Unit<NT> &r, const u32x4 x[4], f32x4 acc[NT],
                                            uint32_t mask_s, uint32_t magic_v, int j0) {
    const bf16x8 neg136 = __builtin_bit_cast(bf16x8, u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, x[2 * e]);
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, x[2 * e + 1]);
        f32x4 c = mfma_bf16_16x16x32(a0, neg136, f32x4{0.f, 0.f, 0.f, 0.f});
        c = mfma_bf16_16x16x32(a1, neg136, c);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 d = mfma_bf16_16x16x32(a0, w16_decode(r.code[j][2 * e], mask_s, magic_v), c);
            d = mfma_bf16_16x16x32(a1, w16_decode(r.code[j][2 * e + 1], mask_s, magic_v), d);
            const uint32_t sbits = NT == 2 ? r.scale[2 * j + e] : (j0 ? r.scale[2 + e] : r.scale[e]);
            const float sc = __uint_as_float(sbits);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = __builtin_fmaf(sc, d[i], acc[j][i]);
        }
    }
}

// One block: 16 NT output columns (both tiles of a unit, or tile j0 of it)
// x `rows` batch rows (rows <= 16); its kW16Waves waves take the K pairs
// w, w + kW16Waves, ... and add their partial sums in LDS. Blocks of one
// tile each double the block count of a skinny layer, which spreads its
// work more evenly over the compute units; two tiles per block share the
// A fragments, which pays once the batch fills the MFMA rows. Dynamic LDS: the block's rows of X ([rows][K] bf16,
// padded to whole KB). MFMA rows past the block's rows read the last row's
// X and are never stored (each output row depends on its own A row only).
template <int kW16Waves, int NT>
__global__ __launch_bounds__(64 * kW16Waves) void w4a16_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ packed,
    const uint16_t *__restrict__ bias, int M, int N, int K, int P, int units, int rows, int m_chunks,
    uint32_t x_lds_bytes, uint32_t mask_s, uint32_t magic_s, uint16_t *__restrict__ Y) {
    extern __shared__ __align__(16) uint8_t xs[];
    __shared__ f32x4 red[kW16Waves][NT][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar offsets
    // blocks of one column pair are adjacent, so the batch chunks of a pair
    // read its weights while they are in L2
    const int tb = (int)(blockIdx.x / (unsigned)m_chunks);
    const int cpair = NT == 2 ? tb : tb >> 1;
    const int j0 = NT == 2 ? 0 : (tb & 1);
    const int m0 = (int)(blockIdx.x % (unsigned)m_chunks) * rows;
    const int rows_here = min(rows, M - m0);

    const __amdgpu_buffer_rsrc_t rw = w16_rsrc(packed, (uint32_t)units * kW16Unit);
    const uint32_t code_off = 16u * (uint32_t)lane + 1024u * (uint32_t)j0;
    const uint32_t scale_off = 2048u + 16u * (uint32_t)(lane & 15);
    const uint32_t unit0 = (uint32_t)cpair * (uint32_t)P * kW16Unit;
    const int xrow = min(lane & 15, rows_here - 1);
    const uint32_t xlane = (uint32_t)xrow * (uint32_t)K * 2u + 16u * (uint32_t)(lane >> 4);
    uint32_t magic_v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "s"(magic_s));

    // A-fragment offsets of unit p, group e: k = 128 p + 64 e + 8 (lane / 16)
    // (+32 for the second step); a group past K (the second of an odd
    // count, whose codes are padding with scale 0) re-reads the first one,
    // so its zero scale multiplies finite values of the same row
    auto x_offsets = [&](int p, uint32_t xoff[2]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int k = 128 * p + 64 * e;  // the same for every lane
            xoff[e] = xlane + 2u * (uint32_t)(k < K ? k : 128 * p);
        }
    };

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int n_iter = wave < P ? (P - wave + kW16Waves - 1) / kW16Waves : 0;
    W16Unit<NT> buf[kW16Depth];

    // X rows m0 .. m0 + rows_here - 1 -> LDS, 1 KB per wave instruction
    // (past the end of X the range check returns zeros), issued together
    // with the first kW16Depth units' weights; the wait for all of them
    // costs little, as the first unit is needed before any compute.
    {
        const __amdgpu_buffer_rsrc_t rx = w16_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
        const uint32_t src0 = (uint32_t)m0 * (uint32_t)K * 2u;
        const int chunks = (int)(((uint32_t)rows_here * (uint32_t)K * 2u + 1023u) / 1024u);
        for (int c = wave; c < chunks; c += kW16Waves)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (w16_lds_void *)(xs + 1024 * c), 16,
                                                     src0 + 1024u * (uint32_t)c + 16u * (uint32_t)lane, 0,
                                                     0, 0);
    }
#pragma unroll
    for (int d = 0; d < kW16Depth; ++d) {
        const int p = min(wave + kW16Waves * d, P - 1);
        w16_load_w<NT>(buf[d], rw, unit0 + (uint32_t)p * kW16Unit, code_off, scale_off);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the copy of X in LDS
    __builtin_amdgcn_s_barrier();
    // unit it of this wave: weights from the ring, A fragments from LDS
    // (read just before use: LDS latency is short)
    auto step = [&](const W16Unit<NT> &u, int it) {
        uint32_t xoff[2];
        x_offsets(wave + kW16Waves * it, xoff);
        u32x4 x[4];
        w16_load_x(x, xs, xoff);
        w16_compute<NT>(u, x, acc, mask_s, magic_v, j0);
    };
    // full rounds: straight-line code, so the loads of the next round stay in
    // flight while this round computes
    int it = 0;
    for (; it + kW16Depth <= n_iter; it += kW16Depth) {
#pragma unroll
        for (int d = 0; d < kW16Depth; ++d) {
            step(buf[d], it + d);
            const int p = min(wave + kW16Waves * (it + d + kW16Depth), P - 1);
            w16_load_w<NT>(buf[d], rw, unit0 + (uint32_t)p * kW16Unit, code_off, scale_off);
        }
    }
#pragma unroll
    for (int d = 0; d < kW16Depth - 1; ++d)
        if (it + d < n_iter) step(buf[d], it + d);

#pragma unroll
    for (int j = 0; j < NT; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    // NT tiles x 16 rows x 16 columns; consecutive threads take consecutive
    // columns of one output row
#pragma unroll
    for (int idx = threadIdx.x; idx < 256 * NT; idx += 64 * kW16Waves) {
        const int j = idx >> 8;
        const int r = (idx >> 4) & 15;
        const int c = idx & 15;
        const int src = 16 * (r >> 2) + c;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < kW16Waves; ++w) v += red[w][j][src][r & 3];
        const int n = 32 * cpair + 16 * (j0 + j) + c;
        if (r < rows_here && n < N) {
            if (bias) v += bf16_bits_to_f32(bias[n]);
            Y[(size_t)(m0 + r) * N + n] = (uint16_t)f32_to_bf16_bits(v);
        }
    }
}

// LDS bytes of X per block: rows x K bf16, rounded up to whole KB (the copy
// moves 1 KB per wave instruction).
uint32_t x_lds_bytes(int rows, int K) { return ((uint32_t)rows * (uint32_t)K * 2u + 1023u) / 1024u * 1024u; }

}  // namespace

// Rows of X per block: at most 16, and as many as fit in the dynamic LDS
// budget; 0 when not even one row of K fits.
int w4a16_rows_per_block(int M, int K) {
    int rows = min(kW16Rows, M);
    while (rows > 0 && x_lds_bytes(rows, K) > kW16LdsMax) --rows;
    return rows;
}

hipError_t launch_w4a16_linear(const uint16_t *X, const uint8_t *packed, const uint16_t *bias, int M,
                               int N, int K, uint16_t *Y, hipStream_t stream) {
    const int P = (K / SVDQ_GROUP + 1) / 2;
    const int rows = w4a16_rows_per_block(M, K);
    const int m_chunks = (M + rows - 1) / rows;
    const int cpairs = (N + 31) / 32;
    const uint32_t xb = x_lds_bytes(rows, K);
    const int units = cpairs * P;
    if (rows <= 8) {
        // a skinny batch: one 16-column tile per block
        const unsigned blocks = (unsigned)((int64_t)2 * cpairs * m_chunks);
        hipLaunchKernelGGL((w4a16_kernel<4, 1>), dim3(blocks), dim3(256), xb, stream, X, packed, bias, M, N, K, P,
                           units, rows, m_chunks, xb, 0x000F000Fu, 0x43004300u, Y);
    } else {
        const int64_t blocks = (int64_t)cpairs * m_chunks;
        // fewer blocks than compute units: split K over more waves per block
        if (blocks < 256 && P >= 16)
            hipLaunchKernelGGL((w4a16_kernel<8, 2>), dim3((unsigned)blocks), dim3(512), xb, stream, X, packed,
                               bias, M, N, K, P, units, rows, m_chunks, xb, 0x000F000Fu, 0x43004300u, Y);
        else
            hipLaunchKernelGGL((w4a16_kernel<4, 2>), dim3((unsigned)blocks), dim3(256), xb, stream, X, packed,
                               bias, M, N, K, P, units, rows, m_chunks, xb, 0x000F000Fu, 0x43004300u, Y);
    }
    return hipGetLastError();
}

}  // namespace svdq
