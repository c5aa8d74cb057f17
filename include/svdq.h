/*
 * svdq.h -- C interface of libsvdq.so: the SVDQuant W4A4 linear with its
 * 16-bit low-rank branch (INT4 and MXFP4 variants), the INT8 tensorwise W8A8
 * linear and the W4A16 linear (4-bit weights, 16-bit activations), for AMD
 * Instinct MI355X (gfx950, CDNA4).
 *
 * The method (sources, cited by page title and passage):
 *  [HF-SVDQ]   "Hugging Face встроила Nunchaku в Diffusers: диффузия быстрее на
 *              30%, видеопамяти нужно до 50% меньше" (iitog.ru), method
 *              paragraph: main layers run with 4-bit weights and 4-bit
 *              activations; activation outliers are moved into the weights;
 *              the hardest part of each weight matrix is a separate 16-bit
 *              low-rank branch; the remainder is quantized to 4 bits.
 *              "Nunchaku Lite" paragraph: such svdq_w4a4 layers replace the
 *              attention and MLP projections (INT4 variant), and awq_w4a16
 *              layers (4-bit weights, 16-bit activations) the
 *              precision-sensitive normalization/modulation layers; hardware
 *              paragraph: an unsupported GPU must be refused with a clear
 *              error, never a wrong result.
 *  [KREA-SVDQ] "SVDQuant ускоряет Krea 2 вдвое даже на старых NVIDIA GPU --
 *              INT8/W4A4 вместо бесполезного FP8" (ainews.so), section
 *              "Решение: INT8 и W4A4": INT8 tensorwise and W4A4 + SVDQuant,
 *              low-rank branches compensating quantization error without a
 *              calibration dataset.
 *  [DC-README] "Diffusion Compiler" README (CodeAlexx/diffusion-compiler),
 *              "Compiler" bullet: a grouped INT4 ("int4-group") physical
 *              weight format.
 *
 *  y = dequant(Q4(X / s) . Q4(R)) + (X / s) . L1 . L2 + bias,
 *  R = diag(s) W - L1 L2   (all on the stored bf16 factors).
 *
 * Conventions for every entry point
 *  - Matrices are row-major. X is [M, K] (tokens x input features); the
 *    weight W is [K, N] (y = X W); bf16 values travel as uint16_t bit
 *    patterns.
 *  - HOST entry points take host pointers, run synchronously on the calling
 *    thread and touch no GPU.
 *  - DEVICE entry points take device pointers (e.g. torch tensors' data),
 *    enqueue kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    return without synchronizing. The library never allocates, frees or
 *    synchronizes device memory; the caller owns every buffer.
 *  - Every check that can be made before a launch is made before the launch.
 *    A failed check returns its status and launches nothing, so no output is
 *    partially written. After launching, a HIP launch error is returned as
 *    SVDQ_ERR_HIP.
 *  - Device pointers must be 16-byte aligned (SVDQ_ERR_MISALIGNED).
 *  - Only gfx950 is served: any other device gives
 *    SVDQ_ERR_UNSUPPORTED_DEVICE before anything is launched.
 *  - Calls on different streams may run concurrently; the library keeps no
 *    mutable state apart from a per-device architecture cache and the fixed
 *    per-device scratch array of svdq_quantize_act_noalloc (the one entry
 *    point whose concurrent calls on a device must be serialized).
 *
 * Codes lie in [-7, 7] (symmetric grid; -8 never produced); qx and qw hold
 * them in one of two containers (svdq_qformat below). Group scales are fp32,
 * group size G = 64 along K, stored group-major.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum svdq_status {
    SVDQ_OK = 0,
    SVDQ_ERR_INVALID_ARGUMENT = 1,  /* null pointer, negative size, bad enum */
    SVDQ_ERR_UNSUPPORTED_SHAPE = 2, /* K % 64, N % 8, rank range, group != 64 */
    SVDQ_ERR_UNSUPPORTED_DEVICE = 3,/* no GPU, or not gfx950 */
    SVDQ_ERR_MISALIGNED = 4,        /* device pointer not 16-byte aligned */
    SVDQ_ERR_NUMERICAL = 5,         /* non-finite weight, SVD failed to converge */
    SVDQ_ERR_HIP = 6                /* a HIP runtime call or launch failed */
} svdq_status;

typedef enum svdq_dtype {
    SVDQ_BF16 = 0,
    SVDQ_F32 = 1
} svdq_dtype;

/* Containers for the INT4 codes (values -7..7) of qx and qw. Both hold the
 * same codes; they differ only in bit layout.
 *  SVDQ_QFMT_INT4: K/2 bytes per row; two's-complement nibbles, byte j holds
 *      k = 2j (low nibble) and k = 2j + 1 (high nibble). The compact,
 *      canonical layout; its GEMM unpacks nibbles to int8 for i8 MFMA.
 *  SVDQ_QFMT_FP6: 3K/4 bytes per row (rows * 3K/4 bytes in all), 48 per
 *      row and group of 64 codes, arranged for coalesced tile loads:
 *      - Rows go in blocks of 128; block b holds rows 128b .. 128b + n_b - 1
 *        with n_b = min(128, rows - 128b) and starts at byte 128 b (3K/4).
 *      - Inside a block the groups follow one another: group g of block b
 *        starts at byte 128 b (3K/4) + g n_b 48, and its row r (0 <= r <
 *        n_b) at + 48 r. So 128 rows x 2 groups of a block are contiguous.
 *      - One row's group is 48 bytes: each code c is an FP6 E2M3 number
 *        equal to c / 8 (bit 5 = sign, bits 0-2 = |c|, exponent field 0);
 *        the codes of half h (k = 32h .. 32h + 31) are packed into 24 bytes
 *        H_h, code k in bits [6(k - 32h), +6) least significant bit first;
 *        the 48 bytes are H_0[0:16] | H_1[0:16] | H_0[16:24] | H_1[16:24]
 *        (three 16-byte planes, the third holding both halves' tails).
 *      Every INT4 code is exact in this form; gfx950's FP6 MFMA, which runs
 *      at twice the int8 rate, reads a half as one 16-byte and one 8-byte
 *      piece and returns each group's partial sum as an exact fp32 integer.
 *      The layout depends on the total row count: a buffer of `rows` rows is
 *      read and written as a whole (no sub-range of rows is a valid buffer).
 */
typedef enum svdq_qformat {
    SVDQ_QFMT_INT4 = 0,
    SVDQ_QFMT_FP6 = 1
} svdq_qformat;

#define SVDQ_GROUP 64
#define SVDQ_MAX_RANK 64

/* Text of a status code (static storage; never NULL). */
const char *svdq_status_string(int status);

/* Library ABI version (bumped on any signature or layout change). */
int svdq_version(void);

/* Bytes per row of packed codes for K codes in container `qfmt` (0 on a bad
 * argument): K/2 for SVDQ_QFMT_INT4, 3K/4 for SVDQ_QFMT_FP6. */
size_t svdq_qrow_bytes(int K, int qfmt);

/* Fail-closed capability check [HF-SVDQ, hardware paragraph]: SVDQ_OK when
 * `device` exists and is gfx950, SVDQ_ERR_UNSUPPORTED_DEVICE otherwise. */
svdq_status svdq_check_device(int device);

/* ---------------------------------------------------------------- HOST --- */

/* Offline preparation of one SVDQuant weight [HF-SVDQ method; KREA-SVDQ
 * "Решение"; DC-README int4-group]:
 *   s_k = fp32(a_k^alpha / w_k^(1-alpha)), a_k = act_absmax[k],
 *         w_k = max_n |W[k, n]|, s_k = 1 if a_k or w_k is 0;
 *   W_hat = diag(s) W; its top-`rank` singular triplets (own subspace
 *   iteration + Jacobi, float64) give L1s = bf16(diag(1/s) U_r Sigma_r^1/2)
 *   and L2 = bf16(Sigma_r^1/2 V_r^T);
 *   R = fp32(s_k (W - L1s L2)) and its INT4 group codes, as in
 *   svdq_prepare_residual.
 * In:  W [K, N] bf16 bits; act_absmax [K] (max |X| per input channel of
 *      calibration activations, e.g. from svdq_channel_absmax); alpha in
 *      [0, 1]; 0 <= rank <= min(64, K, N), rank % 16 == 0; group == 64;
 *      K % 64 == 0, N % 8 == 0.
 * Out: smooth [K] fp32; l1t [rank, K] bf16 bits (L1s transposed: one row per
 *      rank component); l2t [N, rank] bf16 bits (L2 transposed: one row per
 *      output column); qw [N, K/2] packed INT4 (one row per output column);
 *      sw [K/64, N] fp32; sigma [rank] float64 (the singular values used) or
 *      NULL. l1t/l2t may be NULL when rank == 0.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, NUMERICAL (non-finite W or
 *      act_absmax, or the SVD did not converge). Outputs are undefined on
 *      error. */
svdq_status svdq_prepare_weights(const uint16_t *W, int K, int N,
                                 const float *act_absmax, float alpha,
                                 int rank, int group,
                                 float *smooth, uint16_t *l1t, uint16_t *l2t,
                                 uint8_t *qw, float *sw, double *sigma);

/* The residual and weight-quantization half of svdq_prepare_weights, given
 * smoothing factors and bf16 low-rank factors [HF-SVDQ method]:
 *   D[k, n] = sum_{j=0}^{rank-1} L1s[k, j] L2[j, n]   (float64, j ascending)
 *   R[k, n] = fp32(s_k * (W[k, n] - D[k, n]))          (float64, then fp32)
 *   per output column n and K-group g: A = max |R|, sw = fp32(A / 7),
 *   q = clamp(round-half-even(fp32(R / sw)), -7, 7); A == 0 -> sw = 0, q = 0.
 * In:  W [K, N] bf16 bits; smooth [K]; l1t [rank, K]; l2t [N, rank].
 * Out: qw [N, K/2] packed; sw [K/64, N].
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, NUMERICAL. */
svdq_status svdq_prepare_residual(const uint16_t *W, int K, int N,
                                  const float *smooth, const uint16_t *l1t,
                                  const uint16_t *l2t, int rank, int group,
                                  uint8_t *qw, float *sw);

/* INT8 tensorwise weight preparation [KREA-SVDQ "Решение", INT8 tensorwise]:
 *   sw = fp32(max |W| / 127); q = clamp(round-half-even(fp32(W / sw)),
 *   -127, 127); all-zero W -> sw = 0, q = 0.
 * In:  W [K, N] bf16 bits. Out: qw [N, K] int8 (one row per output column,
 *      K contiguous); *sw. Errors: INVALID_ARGUMENT, NUMERICAL. */
svdq_status w8a8_prepare_weights(const uint16_t *W, int K, int N,
                                 int8_t *qw, float *sw);

/* ------------------------------------------------ MXFP4 variant (HOST) --- */

/* The 4-bit float variant of the svdq_w4a4 linear [HF-SVDQ "Nunchaku Lite"
 * paragraph: INT4 and NVFP4 variants; hardware paragraph: the float variant
 * runs on GPUs with native 4-bit float matrix units]. gfx950's native 4-bit
 * float format is OCP MXFP4, so the variant is built as MXFP4: FP4 E2M1
 * codes with one power-of-two E8M0 scale per block of 32 values along K.
 * Smoothing, the low-rank branch, T and the residual R are those of the INT4
 * variant (svdq_prepare_weights gives s, l1t, l2t).
 *   block of 32 (a row of X_hat or a column of R along K): amax = max |v|,
 *   e = floor(log2 amax) - 2 clamped to [-127, 127] (-127 if amax == 0),
 *   E8M0 byte e + 127; code = E2M1 of v / 2^e, round to nearest, ties to the
 *   even mantissa, saturating at 6, a zero result as +0. E2M1: bit 3 sign,
 *   magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7.
 * MX code container (qx, qw) of `rows` rows, rows * K/2 bytes: rows in blocks
 *   of 128 (n_b = min(128, rows - 128b) in block b), block b at byte
 *   128 b K/2; group g (64 k, two blocks of 32) of the block at + g n_b 32;
 *   its half h (the 32-block 2g + h) at + h n_b 16; row r of the block at
 *   + 16 r: 16 bytes, code i of the block in bits [4i, 4i + 4) (byte i / 2,
 *   low nibble for even i). A buffer is only valid as a whole.
 * MX scale matrix (ux, uw): E8M0 bytes [K/32][ld], ld = svdq_mx_scale_ld(rows)
 *   (rows rounded up to a multiple of 16; the padding is never used). */

/* Row stride ld of an MX scale matrix for `rows` rows (0 if rows < 0). */
size_t svdq_mx_scale_ld(int rows);

/* MXFP4 residual of one weight: R = fp32(s_k (W - L1s L2)) exactly as in
 * svdq_prepare_residual, each output column's K values quantized in blocks
 * of 32 as above.
 * In:  W [K, N] bf16 bits; smooth [K]; l1t [rank, K]; l2t [N, rank] (NULL if
 *      rank 0). K % 64 == 0, N % 8 == 0, rank % 16 == 0, rank <= 64.
 * Out: qw: MX code container of N rows (N * K/2 bytes); uw [K/32][ld(N)].
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, NUMERICAL. */
svdq_status svdq_mx_prepare_residual(const uint16_t *W, int K, int N,
                                     const float *smooth, const uint16_t *l1t,
                                     const uint16_t *l2t, int rank,
                                     uint8_t *qw, uint8_t *uw);

/* Bytes of the W4A16 weight container for a [K, N] weight (0 on a bad
 * argument: K <= 0, N <= 0 or K % 64). */
size_t w4a16_weight_bytes(int K, int N);

/* W4A16 weight preparation -- the awq_w4a16 layer type [HF-SVDQ "Nunchaku
 * Lite" paragraph: 4-bit weights with 16-bit activations]. The weight is
 * quantized with the same INT4 grid as the SVDQuant residual, applied to W
 * itself (no smoothing, no low-rank branch; AWQ's activation-aware channel
 * scales, chosen from calibration data, belong to the layer before):
 *   per output column n and K-group g: A = max |W|, sw = fp32(A / 7),
 *   q = clamp(round-half-even(fp32(W / sw)), -7, 7); A == 0 -> sw = 0, q = 0.
 * Out: `packed`, w4a16_weight_bytes(K, N) bytes, laid out for the device
 * kernel's coalesced stream (the layout is part of the ABI):
 *  - columns in pairs of 16-column tiles, C = ceil(N / 32) pairs; K in pairs
 *    of groups, P = ceil(K / 128); unit (b, p) of 2304 bytes at byte
 *    (b P + p) 2304;
 *  - unit bytes [1024 j, 1024 j + 1024) hold tile j (j = 0, 1) as 64 slots
 *    of 16 bytes; dword d (0..3) of slot l holds column n = 32b + 16j +
 *    l % 16 at k = 64(2p + d / 2) + 32(d % 2) + 8(l / 16) + i, i = 0..7,
 *    each code as the nibble u = q + 8 (1..15), i = 2t in bits [4t, 4t + 4)
 *    and i = 2t + 1 in bits [16 + 4t, 20 + 4t);
 *  - unit bytes [2048, 2304): fp32 sw of column 32b + 16j + c and group
 *    2p + e at byte 2048 + 16c + 8j + 4e (c = 0..15; j, e = 0..1);
 *  - columns n >= N and groups g >= K/64 are padding: u = 8, sw = 0.
 * In: W [K, N] bf16 bits (host), group == 64, K % 64 == 0, N >= 1.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, NUMERICAL (non-finite W). */
svdq_status w4a16_prepare_weights(const uint16_t *W, int K, int N, int group,
                                  uint8_t *packed);

/* Re-encodes packed codes from the canonical INT4 container into `qfmt`
 * (SVDQ_QFMT_INT4 copies). In: q [rows, K/2]; out: [rows, svdq_qrow_bytes(K,
 * qfmt)]. Host pointers. Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE (K % 64),
 * NUMERICAL (a nibble holding -8, which no SVDQuant code uses). */
svdq_status svdq_repack_codes(const uint8_t *q, int rows, int K, int qfmt,
                              uint8_t *out);

/* -------------------------------------------------------------- DEVICE --- */

/* Calibration statistic for smoothing (self-calibration: the statistic comes
 * from the activations themselves, no dataset) [HF-SVDQ method]:
 *   absmax[k] = max(absmax[k], max_m |X[m, k]|)   (running maximum; the caller
 *   zero-fills absmax before the first batch).
 * In: X [M, K] bf16 (device). In/out: absmax [K] fp32 (device).
 * Order-independent (integer max on the fp32 bit patterns): deterministic.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE (K % 8), MISALIGNED,
 *      UNSUPPORTED_DEVICE, HIP. */
svdq_status svdq_channel_absmax(const uint16_t *X, int M, int K, float *absmax,
                                void *stream);

/* Bytes of the optional device workspace of svdq_quantize_act and
 * svdq_mx_quantize_act for an [M, K] input at this rank (0 when the pass
 * needs none). */
size_t svdq_act_workspace_bytes(int M, int K, int rank);

/* Fused activation quantization -- one pass over X [HF-SVDQ method]:
 *   X_hat = fp32(X / s_k)   (IEEE fp32 division, round to nearest even);
 *   per row m and K-group g: A = max |X_hat|, sx[g, m] = fp32(A / 7),
 *   qx = clamp(round-half-even(fp32(X_hat / sx)), -7, 7) packed to nibbles;
 *   A == 0 -> sx = 0, codes 0;
 *   T[m, :] = bf16(X[m, :] L1s)  -- the low-rank down-projection on raw X with
 *   1/s folded into L1s, fp32 accumulation, one rounding to bf16.
 * In:  X [M, K] bf16; smooth [K] fp32; l1t [rank, K] bf16 (NULL if rank 0);
 *      qfmt: the container of qx (svdq_qformat).
 * Out: qx [M, svdq_qrow_bytes(K, qfmt)]; sx [K/64, M] fp32; T [M, rank] bf16 (NULL if
 *      rank 0). M >= 0 (M == 0 launches nothing), K % 64 == 0,
 *      rank % 16 == 0, rank <= 64, group == 64.
 * Workspace: NULL, or device memory of at least svdq_act_workspace_bytes(M,
 *      K, rank) bytes owned by the caller (not read before it is written):
 *      with it the pass splits K across blocks (fp32 partial sums of T,
 *      combined by a second kernel), which fills the GPU when M is small.
 *      A non-NULL workspace that is too small is INVALID_ARGUMENT.
 * Deterministic: T's partial sums are combined in a fixed order (which
 *      depends only on M, K and whether a workspace is given).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, UNSUPPORTED_DEVICE,
 *      HIP. */
svdq_status svdq_quantize_act(const uint16_t *X, const float *smooth,
                              const uint16_t *l1t, int M, int K, int rank,
                              int group, int qfmt, uint8_t *qx, float *sx,
                              uint16_t *T, void *workspace, size_t workspace_bytes,
                              void *stream);

/* svdq_quantize_act without a caller workspace and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same
 * arguments, results and errors as svdq_quantize_act given a workspace (the
 * same kernels and the same split of K, so the outputs are identical); the
 * fp32 partial sums of T go to a fixed 32 MiB device array inside the
 * library (one per device, held until the process ends; its address is
 * looked up on the first call on each device). Every shape the pass accepts
 * fits it (when K is split in p parts, p * M <= 131072 and rank <= 64); a
 * call that would need more is refused with SVDQ_ERR_UNSUPPORTED_SHAPE
 * before any launch. The array is shared by every call on a device: calls
 * that overlap in time on one device (different streams, threads or
 * processes' shared contexts) race on it and must be serialized by the
 * caller. Nothing in it needs clearing between calls (each call writes
 * every partial it reads).
 * Errors: as svdq_quantize_act, and SVDQ_ERR_HIP if the array's address
 *      cannot be obtained. */
svdq_status svdq_quantize_act_noalloc(const uint16_t *X, const float *smooth,
                                      const uint16_t *l1t, int M, int K,
                                      int rank, int group, int qfmt,
                                      uint8_t *qx, float *sx, uint16_t *T,
                                      void *stream);

/* The W4A4 linear with fused low-rank up-projection and bias
 * [HF-SVDQ method and "Nunchaku Lite" paragraph]:
 *   P[g, m, n] = sum_{k in g} qx[m, k] qw[n, k]      (exact: i8 MFMA for the
 *                                                    INT4 container, FP6 MFMA
 *                                                    for the FP6 container)
 *   acc[m, n]  = sum_g (sx[g, m] sw[g, n]) P[g, m, n] (fp32)
 *   y[m, n]    = acc + sum_j T[m, j] L2[j, n] + bias[n]  (bf16 MFMA, fp32)
 *   Y = y rounded once to bf16 (round to nearest even) or stored as fp32.
 * In:  qx [M, R], sx [K/64, M], T [M, rank] (NULL if rank 0),
 *      qw [N, R], sw [K/64, N], l2t [N, rank] (NULL if rank 0),
 *      bias [N] bf16 or NULL; qfmt: the container of both qx and qw, whose
 *      rows are R = svdq_qrow_bytes(K, qfmt) bytes. y_dtype: SVDQ_BF16 or
 *      SVDQ_F32.
 * Out: Y [M, N] of y_dtype.
 * Shapes: M >= 0, K % 64 == 0, N % 8 == 0, rank % 16 == 0, rank <= 64.
 * Deterministic (no atomics; fixed summation order).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, UNSUPPORTED_DEVICE,
 *      HIP. */
svdq_status svdq_w4a4_linear(const uint8_t *qx, const float *sx,
                             const uint16_t *T, const uint8_t *qw,
                             const float *sw, const uint16_t *l2t,
                             const uint16_t *bias, int M, int N, int K,
                             int rank, int group, int qfmt, void *Y,
                             int y_dtype, void *stream);

/* MLP pair on the device [HF-SVDQ method and "Nunchaku Lite" paragraphs:
 * svdq_w4a4 on the MLP projections, fused kernels]: the up-projection of a
 * DiT MLP whose output goes through GELU into the down-projection. The
 * up-projection is svdq_w4a4_linear on the FP6 container; instead of Y it
 * emits the down-projection's activation side, computed from
 *   y_up = bf16(acc + T L2 + bias)                 (as svdq_w4a4_linear)
 *   g    = bf16(GELU(y_up)),  GELU(y) = y Phi(y) = (y / 2) erfc(-y / sqrt 2),
 *          one correct rounding of the exact value
 * exactly as svdq_quantize_act would from X = g with K_down = N:
 *   qx_down [M, svdq_qrow_bytes(N, SVDQ_QFMT_FP6)] (FP6 container),
 *   sx_down [N/64, M] fp32, T_down [M, rank_down] = bf16(g L1s_down)
 *   (fp32 partial sums per 128 columns, combined in a fixed order).
 * In:  the up-projection's operands as svdq_w4a4_linear with qfmt =
 *      SVDQ_QFMT_FP6 (qx, sx, T, qw, sw, l2t, bias, M, N, K, rank, group);
 *      smooth_down [N] fp32 and l1t_down [rank_down, N] bf16 (NULL if
 *      rank_down is 0): the down-projection's smoothing factors and
 *      transposed low-rank down factor (svdq_prepare_weights of its weight).
 * Out: qx_down, sx_down, T_down (NULL if rank_down is 0); Y_up [M, N] bf16,
 *      the up-projection's output, only if not NULL (for checks; the fused
 *      path does not need it).
 * Workspace: device memory of svdq_mlp_workspace_bytes(M, N, rank_down)
 *      bytes (NULL if that is 0), owned by the caller, not read before it is
 *      written.
 * Shapes: as svdq_w4a4_linear, plus N % 64 == 0 (the down-projection's K),
 *      rank_down % 16 == 0, rank_down <= 64. Deterministic.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, UNSUPPORTED_DEVICE,
 *      HIP. */
size_t svdq_mlp_workspace_bytes(int M, int N, int rank_down);
svdq_status svdq_w4a4_linear_gelu_quantize(const uint8_t *qx, const float *sx, const uint16_t *T,
                                           const uint8_t *qw, const float *sw, const uint16_t *l2t,
                                           const uint16_t *bias, int M, int N, int K, int rank, int group,
                                           const float *smooth_down, const uint16_t *l1t_down, int rank_down,
                                           uint8_t *qx_down, float *sx_down, uint16_t *T_down, uint16_t *Y_up,
                                           void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace w8a8_linear needs for an [M, K] input. */
size_t w8a8_workspace_bytes(int M, int K);

/* INT8 tensorwise W8A8 linear [KREA-SVDQ "Решение", INT8 tensorwise]:
 *   sx = fp32(max |X| / 127) over the whole X (computed on the device by an
 *   order-independent max: deterministic); qx = clamp(round-half-even(
 *   fp32(X / sx)), -127, 127) (all-zero X -> sx = 0, codes 0);
 *   acc[m, n] = sum_k qx[m, k] qw[n, k]  (int32, all of K);
 *   Y = bf16(fp32(acc) * fp32(sx * sw) + bias[n])  (round to nearest even).
 * In:  X [M, K] bf16; qw [N, K] int8; sw (host value); bias [N] bf16 or NULL;
 *      workspace of at least w8a8_workspace_bytes(M, K) bytes (device,
 *      16-byte aligned; holds the int8 codes of X and the scale).
 * Out: Y [M, N] bf16. Shapes: K % 64 == 0, N % 8 == 0, K * 127^2 < 2^31,
 *      M * K < 2^31 and N * K < 2^31.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, UNSUPPORTED_DEVICE,
 *      HIP. */
svdq_status w8a8_linear(const uint16_t *X, const int8_t *qw, float sw,
                        const uint16_t *bias, int M, int N, int K,
                        void *workspace, size_t workspace_bytes, uint16_t *Y,
                        void *stream);

/* Fused activation quantization of the MXFP4 variant -- one pass over X:
 * X_hat = fp32(X / s_k) (IEEE fp32 division, as svdq_quantize_act); per row
 * and block of 32 along K the E8M0 scale and E2M1 codes above;
 * T[m, :] = bf16(X[m, :] L1s) as svdq_quantize_act.
 * In:  X [M, K] bf16; smooth [K]; l1t [rank, K] (NULL if rank 0).
 * Out: qx: MX code container of M rows; ux [K/32][ld(M)] (16-byte aligned);
 *      T [M, rank] bf16 (NULL if rank 0). K % 64 == 0, rank % 16 == 0,
 *      rank <= 64; M == 0 launches nothing.
 * Workspace: as svdq_quantize_act (svdq_act_workspace_bytes).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, UNSUPPORTED_DEVICE,
 *      HIP. */
svdq_status svdq_mx_quantize_act(const uint16_t *X, const float *smooth,
                                 const uint16_t *l1t, int M, int K, int rank,
                                 uint8_t *qx, uint8_t *ux, uint16_t *T,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* The MXFP4 linear with fused low-rank up-projection and bias:
 *   acc[m, n] = sum_b 2^(ex[b, m] + ew[b, n]) sum_{k in b} e2m1(qx) e2m1(qw)
 *               (the scaled FP4 MFMA: block scales applied by the matrix
 *               core, fp32 accumulation over the blocks in ascending order)
 *   y = acc + sum_j T[m, j] L2[j, n] + bias[n]  (bf16 MFMA, fp32)
 *   Y = y rounded once to bf16 (nearest even) or stored as fp32.
 * In:  qx, ux (svdq_mx_quantize_act), T [M, rank]; qw, uw
 *      (svdq_mx_prepare_residual), l2t [N, rank]; bias [N] bf16 or NULL;
 *      y_dtype SVDQ_BF16 or SVDQ_F32.
 * Out: Y [M, N]. Shapes: M >= 0, K % 64 == 0, N % 8 == 0, rank % 16 == 0,
 *      rank <= 64. Deterministic.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, UNSUPPORTED_DEVICE,
 *      HIP. */
svdq_status svdq_mx_linear(const uint8_t *qx, const uint8_t *ux,
                           const uint16_t *T, const uint8_t *qw,
                           const uint8_t *uw, const uint16_t *l2t,
                           const uint16_t *bias, int M, int N, int K,
                           int rank, void *Y, int y_dtype, void *stream);

/* The W4A16 linear [HF-SVDQ "Nunchaku Lite" paragraph, awq_w4a16]:
 *   y[m, n] = sum_g sw[g, n] sum_{k in g} X[m, k] q[k, n] + bias[n]
 *   (bf16 MFMA on the exact bf16 values of X and of the codes, fp32
 *   accumulation per group, fp32 group scaling), rounded once to bf16
 *   (round to nearest even).
 * In:  X [M, K] bf16; packed: the container of w4a16_prepare_weights for
 *      this K and N; bias [N] bf16 or NULL. group == 64.
 * Out: Y [M, N] bf16.
 * Shapes: M >= 0 (M == 0 launches nothing), K % 64 == 0, K <= 28672,
 *      N >= 1 (any N), M * K < 2^30, w4a16_weight_bytes(K, N) < 2^31. Built
 *      for the batch sizes of conditioning inputs: the weight is read once
 *      per block of rows of X (16 rows, fewer once 2 K bytes per row no
 *      longer fit 56 KB of LDS).
 * Deterministic (fixed summation order, no atomics).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_SHAPE, MISALIGNED, UNSUPPORTED_DEVICE,
 *      HIP. */
svdq_status w4a16_linear(const uint16_t *X, const uint8_t *packed,
                         const uint16_t *bias, int M, int N, int K, int group,
                         uint16_t *Y, void *stream);

/* ------------------------------------------- TEST-ONLY (same kernels) --- */

/* The device's GELU rule of svdq_w4a4_linear_gelu_quantize applied
 * elementwise: g[i] = bf16(GELU(y[i])) for n bf16 values (device pointers),
 * so that it can be checked on every bf16 input. n >= 0.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED_DEVICE, HIP. */
svdq_status svdq_debug_gelu_bf16(const uint16_t *y, uint16_t *g, int n, void *stream);

/* INT4 group partials from the W4A4 GEMM's own main loop (container qfmt):
 *   P[g, m, n] = sum_{k in g} qx[m, k] qw[n, k]  as int32, [K/64, M, N]. */
svdq_status svdq_debug_group_partials(const uint8_t *qx, const uint8_t *qw,
                                      int M, int N, int K, int group, int qfmt,
                                      int32_t *P, void *stream);

/* INT8 accumulators from the W8A8 GEMM's own main loop:
 *   acc[m, n] = sum_k qx[m, k] qw[n, k] as int32, [M, N]. */
svdq_status w8a8_debug_acc(const int8_t *qx, const int8_t *qw, int M, int N,
                           int K, int32_t *acc, void *stream);

/* Matrix-core rate on this device, the denominator a roofline fraction can
 * also be quoted against besides the published peak: `blocks` blocks of 4
 * waves each run `iters` rounds of 4 independent MFMAs of one kind (kind 0:
 * FP6 32x32x64 with block scales, 1: int8 32x32x32, 2: bf16 32x32x16) back
 * to back. out (device, 16-byte aligned, 2 * 4 * blocks uint64 values):
 * per wave its span in shader-clock cycles and in ticks of the 100 MHz
 * real-time counter (their ratio is the shader clock under that load).
 * svdq_debug_mfma_ops gives the operations (2 M N K per MFMA) of such a
 * launch (0 on a bad argument).
 * Errors: INVALID_ARGUMENT, MISALIGNED, UNSUPPORTED_DEVICE, HIP. */
int64_t svdq_debug_mfma_ops(int kind, int blocks, int iters);
svdq_status svdq_debug_mfma_rate(int kind, int blocks, int iters, uint64_t *out, void *stream);

/* Test hook for the fail-closed path: when `arch` is non-NULL the device
 * check sees that architecture name instead of the real one (NULL restores
 * the real one). Host-only; never launches anything. */
svdq_status svdq_debug_set_arch_override(const char *arch);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
