// Internal declarations shared by the C-ABI layer, the host preparation code
// and the HIP kernel launchers of libsvdq.so. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "svdq.h"

namespace svdq {

// ---- host preparation (prepare.cpp) ----
svdq_status prepare_weights_impl(const uint16_t *W, int K, int N,
                                 const float *act_absmax, float alpha, int rank,
                                 float *smooth, uint16_t *l1t, uint16_t *l2t,
                                 uint8_t *qw, float *sw, double *sigma);
svdq_status prepare_residual_impl(const uint16_t *W, int K, int N,
                                  const float *smooth, const uint16_t *l1t,
                                  const uint16_t *l2t, int rank, uint8_t *qw,
                                  float *sw);
svdq_status w8a8_prepare_impl(const uint16_t *W, int K, int N, int8_t *qw, float *sw);
svdq_status mx_prepare_residual_impl(const uint16_t *W, int K, int N, const float *smooth,
                                     const uint16_t *l1t, const uint16_t *l2t, int rank, uint8_t *qw,
                                     uint8_t *uw);
size_t mx_scale_ld(int rows);
svdq_status w4a16_prepare_impl(const uint16_t *W, int K, int N, uint8_t *packed);
size_t w4a16_container_bytes(int K, int N);
svdq_status repack_codes_impl(const uint8_t *q, int rows, int K, int qfmt, uint8_t *out);
svdq_status truncated_svd(const double *A, int K, int N, int rank, double *U,
                          double *S, double *V);
bool all_finite_bf16(const uint16_t *p, int64_t n);

// ---- device launchers (act_quant.hip, w4a4_gemm.hip, w4a4_fp6_gemm.hip, w8a8.hip, w4a16.hip,
//      mx_gemm.hip) ----
// Arguments are validated by the caller; launchers only pick a grid and launch.
hipError_t launch_channel_absmax(const uint16_t *X, int M, int K, float *absmax,
                                 hipStream_t stream);
// activation passes: workspace (nullable) holds act_workspace_size(M, K,
// rank) bytes for T's fp32 partials when K is split across blocks
int act_k_parts(int M, int K);
size_t act_workspace_size(int M, int K, int rank);
// fixed device scratch of svdq_quantize_act_noalloc (bytes; covers
// act_workspace_size for every supported shape) and its address on the
// current device, looked up once per device
constexpr size_t kActScratchBytes = (size_t)32 << 20;
hipError_t act_scratch_pointer(float **out);
hipError_t launch_quantize_act(const uint16_t *X, const float *smooth,
                               const uint16_t *l1t, int M, int K, int rank,
                               int qfmt, uint8_t *qx, float *sx, uint16_t *T,
                               float *workspace, hipStream_t stream);
hipError_t launch_w4a4_linear(const uint8_t *qx, const float *sx,
                              const uint16_t *T, const uint8_t *qw,
                              const float *sw, const uint16_t *l2t,
                              const uint16_t *bias, int M, int N, int K,
                              int rank, void *Y, bool y_f32, hipStream_t stream);
hipError_t launch_w4a4_partials(const uint8_t *qx, const uint8_t *qw, int M,
                                int N, int K, int32_t *P, hipStream_t stream);
hipError_t launch_w4a4_fp6_linear(const uint8_t *qx, const float *sx,
                                  const uint16_t *T, const uint8_t *qw,
                                  const float *sw, const uint16_t *l2t,
                                  const uint16_t *bias, int M, int N, int K,
                                  int rank, void *Y, bool y_f32, hipStream_t stream);
hipError_t launch_w4a4_fp6_partials(const uint8_t *qx, const uint8_t *qw, int M,
                                    int N, int K, int32_t *P, hipStream_t stream);
// What the fused MLP epilogue emits for the down-projection (K_down = N of
// the up-projection): FP6 codes qx [M rows, N], group scales sx [N / 64, M],
// fp32 partial sums tpart [tiles_n][M][rank] of g L1s over each 128-column
// tile, and optionally the bf16 up-projection output y_up [M, N].
struct MlpOut {
    const float *smooth;  // [N] smoothing factors of the down-projection
    const uint16_t *l1t;  // [rank, N] its low-rank down factor, transposed
    int rank;
    uint8_t *qx;
    float *sx;
    float *tpart;
    uint16_t *y_up;       // may be null
};
int mlp_tiles_n(int N);
hipError_t launch_w4a4_fp6_mlp(const uint8_t *qx, const float *sx, const uint16_t *T, const uint8_t *qw,
                               const float *sw, const uint16_t *l2t, const uint16_t *bias, int M, int N, int K,
                               int rank, const MlpOut &out, hipStream_t stream);
hipError_t launch_tpart_reduce(const float *tpart, int parts, int M, int rank, uint16_t *T, hipStream_t stream);
hipError_t launch_gelu_bf16(const uint16_t *y, uint16_t *g, int n, hipStream_t stream);
hipError_t launch_w8a8_linear(const uint16_t *X, const int8_t *qw, float sw,
                              const uint16_t *bias, int M, int N, int K,
                              void *workspace, uint16_t *Y, hipStream_t stream);
hipError_t launch_w8a8_acc(const int8_t *qx, const int8_t *qw, int M, int N,
                           int K, int32_t *acc, hipStream_t stream);
size_t w8a8_workspace_size(int M, int K);
int w4a16_rows_per_block(int M, int K);
hipError_t launch_mx_quantize_act(const uint16_t *X, const float *smooth, const uint16_t *l1t, int M,
                                  int K, int rank, uint8_t *qx, uint8_t *ux, uint16_t *T, float *workspace,
                                  hipStream_t stream);
hipError_t launch_mx_linear(const uint8_t *qx, const uint8_t *ux, const uint16_t *T, const uint8_t *qw,
                            const uint8_t *uw, const uint16_t *l2t, const uint16_t *bias, int M, int N, int K,
                            int rank, void *Y, bool y_f32, hipStream_t stream);
hipError_t launch_w4a16_linear(const uint16_t *X, const uint8_t *packed, const uint16_t *bias, int M,
                               int N, int K, uint16_t *Y, hipStream_t stream);

// matrix-core rate microbenchmark (peak.hip)
int64_t mfma_rate_ops_per_wave_round(int kind);
hipError_t launch_mfma_rate(int kind, int blocks, int iters, uint64_t *out, hipStream_t stream);

}  // namespace svdq
