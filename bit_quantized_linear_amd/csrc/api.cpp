// C-ABI layer of libsvdq.so: argument validation, the fail-closed device
// check and launch dispatch. Every check runs before anything is launched, so
// a rejected call writes nothing: an unsupported device or argument fails
// closed with a status instead of producing output ("Hugging Face встроила
// Nunchaku в Diffusers..." (iitog.ru), hardware paragraph).

#include "svdq.h"
#include "internal.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>

namespace {

constexpr int kAbiVersion = 8;
constexpr int kMaxDevices = 64;

std::mutex g_mutex;
int g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
bool g_override_set = false;
std::string g_override_arch;

bool is_gfx950(const char *name) {
    // gcnArchName looks like "gfx950:sramecc+:xnack-"
    return std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':');
}

svdq_status device_ok(int device) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_override_set) return is_gfx950(g_override_arch.c_str()) ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
    if (device < 0 || device >= kMaxDevices) return SVDQ_ERR_UNSUPPORTED_DEVICE;
    if (g_arch_state[device] == 0) {
        int count = 0;
        if (hipGetDeviceCount(&count) != hipSuccess || device >= count) {
            (void)hipGetLastError();
            return SVDQ_ERR_UNSUPPORTED_DEVICE;
        }
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
            (void)hipGetLastError();
            return SVDQ_ERR_UNSUPPORTED_DEVICE;
        }
        g_arch_state[device] = is_gfx950(prop.gcnArchName) ? 1 : 2;
    }
    return g_arch_state[device] == 1 ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
}

svdq_status current_device_ok() {
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (g_override_set) return is_gfx950(g_override_arch.c_str()) ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return SVDQ_ERR_UNSUPPORTED_DEVICE;
    }
    return device_ok(dev);
}

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

svdq_status launched(hipError_t e) {
    if (e != hipSuccess) return SVDQ_ERR_HIP;
    e = hipGetLastError();
    return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP;
}

// Buffer loads address each operand with 32-bit offsets.
bool fits_buffer(int64_t rows, int64_t row_bytes) { return rows * row_bytes < ((int64_t)1 << 31); }

// Shape rules shared by the W4A4 entry points.
svdq_status check_w4a4_shape(int M, int K, int rank, int group) {
    if (M < 0 || K <= 0 || rank < 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (group != SVDQ_GROUP) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (K % SVDQ_GROUP != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rank > SVDQ_MAX_RANK || rank % 16 != 0) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    return SVDQ_OK;
}

}  // namespace

extern "C" {

const char *svdq_status_string(int status) {
    switch (status) {
        case SVDQ_OK: return "ok";
        case SVDQ_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SVDQ_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case SVDQ_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        case SVDQ_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case SVDQ_ERR_NUMERICAL: return "numerical failure (non-finite input or SVD did not converge)";
        case SVDQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int svdq_version(void) { return kAbiVersion; }

size_t svdq_qrow_bytes(int K, int qfmt) {
    if (K <= 0 || K % SVDQ_GROUP) return 0;
    if (qfmt == SVDQ_QFMT_INT4) return (size_t)K / 2;
    if (qfmt == SVDQ_QFMT_FP6) return (size_t)K / 4 * 3;
    return 0;
}

svdq_status svdq_check_device(int device) { return device_ok(device); }

svdq_status svdq_debug_set_arch_override(const char *arch) {
    std::lock_guard<std::mutex> lock(g_mutex);
    if (arch) {
        g_override_set = true;
        g_override_arch = arch;
    } else {
        g_override_set = false;
        g_override_arch.clear();
    }
    return SVDQ_OK;
}

// ------------------------------------------------------------------ host ---

svdq_status svdq_prepare_weights(const uint16_t *W, int K, int N,
                                 const float *act_absmax, float alpha,
                                 int rank, int group, float *smooth,
                                 uint16_t *l1t, uint16_t *l2t, uint8_t *qw,
                                 float *sw, double *sigma) {
    if (!W || !act_absmax || !smooth || !qw || !sw) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K <= 0 || N <= 0 || rank < 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SVDQ_ERR_INVALID_ARGUMENT;
    if (group != SVDQ_GROUP || K % SVDQ_GROUP || N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rank > SVDQ_MAX_RANK || rank % 16 || rank > K || rank > N) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rank > 0 && (!l1t || !l2t)) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!svdq::all_finite_bf16(W, (int64_t)K * N)) return SVDQ_ERR_NUMERICAL;
    for (int k = 0; k < K; ++k)
        if (!std::isfinite(act_absmax[k]) || act_absmax[k] < 0.0f) return SVDQ_ERR_NUMERICAL;
    return svdq::prepare_weights_impl(W, K, N, act_absmax, alpha, rank, smooth, l1t, l2t, qw, sw, sigma);
}

svdq_status svdq_prepare_residual(const uint16_t *W, int K, int N,
                                  const float *smooth, const uint16_t *l1t,
                                  const uint16_t *l2t, int rank, int group,
                                  uint8_t *qw, float *sw) {
    if (!W || !smooth || !qw || !sw) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K <= 0 || N <= 0 || rank < 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (group != SVDQ_GROUP || K % SVDQ_GROUP || N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rank > SVDQ_MAX_RANK || rank % 16 || rank > K || rank > N) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rank > 0 && (!l1t || !l2t)) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!svdq::all_finite_bf16(W, (int64_t)K * N)) return SVDQ_ERR_NUMERICAL;
    if (rank > 0 && (!svdq::all_finite_bf16(l1t, (int64_t)rank * K) ||
                     !svdq::all_finite_bf16(l2t, (int64_t)rank * N)))
        return SVDQ_ERR_NUMERICAL;
    for (int k = 0; k < K; ++k)
        if (!std::isfinite(smooth[k]) || !(smooth[k] > 0.0f)) return SVDQ_ERR_NUMERICAL;
    return svdq::prepare_residual_impl(W, K, N, smooth, l1t, l2t, rank, qw, sw);
}

svdq_status svdq_repack_codes(const uint8_t *q, int rows, int K, int qfmt, uint8_t *out) {
    if (rows < 0 || K <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (qfmt != SVDQ_QFMT_INT4 && qfmt != SVDQ_QFMT_FP6) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K % SVDQ_GROUP) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rows > 0 && (!q || !out)) return SVDQ_ERR_INVALID_ARGUMENT;
    return svdq::repack_codes_impl(q, rows, K, qfmt, out);
}

svdq_status w8a8_prepare_weights(const uint16_t *W, int K, int N, int8_t *qw, float *sw) {
    if (!W || !qw || !sw || K <= 0 || N <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!svdq::all_finite_bf16(W, (int64_t)K * N)) return SVDQ_ERR_NUMERICAL;
    return svdq::w8a8_prepare_impl(W, K, N, qw, sw);
}

size_t w4a16_weight_bytes(int K, int N) {
    if (K <= 0 || N <= 0 || K % SVDQ_GROUP) return 0;
    return svdq::w4a16_container_bytes(K, N);
}

svdq_status w4a16_prepare_weights(const uint16_t *W, int K, int N, int group, uint8_t *packed) {
    if (!W || !packed || K <= 0 || N <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (group != SVDQ_GROUP || K % SVDQ_GROUP) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!svdq::all_finite_bf16(W, (int64_t)K * N)) return SVDQ_ERR_NUMERICAL;
    return svdq::w4a16_prepare_impl(W, K, N, packed);
}

size_t svdq_mx_scale_ld(int rows) { return rows < 0 ? 0 : svdq::mx_scale_ld(rows); }

svdq_status svdq_mx_prepare_residual(const uint16_t *W, int K, int N, const float *smooth,
                                     const uint16_t *l1t, const uint16_t *l2t, int rank, uint8_t *qw,
                                     uint8_t *uw) {
    if (!W || !smooth || !qw || !uw) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K <= 0 || N <= 0 || rank < 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K % SVDQ_GROUP || N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rank > SVDQ_MAX_RANK || rank % 16 || rank > K || rank > N) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (rank > 0 && (!l1t || !l2t)) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!svdq::all_finite_bf16(W, (int64_t)K * N)) return SVDQ_ERR_NUMERICAL;
    if (rank > 0 && (!svdq::all_finite_bf16(l1t, (int64_t)rank * K) ||
                     !svdq::all_finite_bf16(l2t, (int64_t)rank * N)))
        return SVDQ_ERR_NUMERICAL;
    for (int k = 0; k < K; ++k)
        if (!std::isfinite(smooth[k]) || !(smooth[k] > 0.0f)) return SVDQ_ERR_NUMERICAL;
    return svdq::mx_prepare_residual_impl(W, K, N, smooth, l1t, l2t, rank, qw, uw);
}

// ---------------------------------------------------------------- device ---

svdq_status svdq_channel_absmax(const uint16_t *X, int M, int K, float *absmax, void *stream) {
    if (!absmax || M < 0 || K <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (M > 0 && !X) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(X) || !aligned16(absmax)) return SVDQ_ERR_MISALIGNED;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    return launched(svdq::launch_channel_absmax(X, M, K, absmax, (hipStream_t)stream));
}

size_t svdq_act_workspace_bytes(int M, int K, int rank) {
    if (M < 0 || K <= 0 || K % SVDQ_GROUP || rank < 0) return 0;
    return svdq::act_workspace_size(M, K, rank);
}

svdq_status svdq_quantize_act(const uint16_t *X, const float *smooth,
                              const uint16_t *l1t, int M, int K, int rank,
                              int group, int qfmt, uint8_t *qx, float *sx,
                              uint16_t *T, void *workspace, size_t workspace_bytes, void *stream) {
    svdq_status st = check_w4a4_shape(M, K, rank, group);
    if (st != SVDQ_OK) return st;
    if (qfmt != SVDQ_QFMT_INT4 && qfmt != SVDQ_QFMT_FP6) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!smooth || (M > 0 && (!X || !qx || !sx))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (rank > 0 && (!l1t || (M > 0 && !T))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (workspace && workspace_bytes < svdq::act_workspace_size(M, K, rank)) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(X) || !aligned16(smooth) || !aligned16(l1t) || !aligned16(qx) ||
        !aligned16(sx) || !aligned16(T) || !aligned16(workspace))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    return launched(svdq::launch_quantize_act(X, smooth, rank ? l1t : nullptr, M, K, rank, qfmt, qx, sx,
                                              rank ? T : nullptr, static_cast<float *>(workspace),
                                              (hipStream_t)stream));
}

svdq_status svdq_quantize_act_noalloc(const uint16_t *X, const float *smooth, const uint16_t *l1t, int M,
                                      int K, int rank, int group, int qfmt, uint8_t *qx, float *sx,
                                      uint16_t *T, void *stream) {
    svdq_status st = check_w4a4_shape(M, K, rank, group);
    if (st != SVDQ_OK) return st;
    if (qfmt != SVDQ_QFMT_INT4 && qfmt != SVDQ_QFMT_FP6) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!smooth || (M > 0 && (!X || !qx || !sx))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (rank > 0 && (!l1t || (M > 0 && !T))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (svdq::act_workspace_size(M, K, rank) > svdq::kActScratchBytes) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(X) || !aligned16(smooth) || !aligned16(l1t) || !aligned16(qx) || !aligned16(sx) ||
        !aligned16(T))
        return SVDQ_ERR_MISALIGNED;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    float *scratch = nullptr;
    if (svdq::act_scratch_pointer(&scratch) != hipSuccess) return SVDQ_ERR_HIP;
    return launched(svdq::launch_quantize_act(X, smooth, rank ? l1t : nullptr, M, K, rank, qfmt, qx, sx,
                                              rank ? T : nullptr, scratch, (hipStream_t)stream));
}

size_t svdq_mlp_workspace_bytes(int M, int N, int rank_down) {
    if (M < 0 || N <= 0 || rank_down < 0) return 0;
    return (size_t)svdq::mlp_tiles_n(N) * (size_t)M * (size_t)rank_down * sizeof(float);
}

svdq_status svdq_w4a4_linear_gelu_quantize(const uint8_t *qx, const float *sx, const uint16_t *T,
                                           const uint8_t *qw, const float *sw, const uint16_t *l2t,
                                           const uint16_t *bias, int M, int N, int K, int rank, int group,
                                           const float *smooth_down, const uint16_t *l1t_down, int rank_down,
                                           uint8_t *qx_down, float *sx_down, uint16_t *T_down, uint16_t *Y_up,
                                           void *workspace, size_t workspace_bytes, void *stream) {
    svdq_status st = check_w4a4_shape(M, K, rank, group);
    if (st != SVDQ_OK) return st;
    if (N <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    st = check_w4a4_shape(M, N, rank_down, group);  // the down-projection's K is N
    if (st != SVDQ_OK) return st;
    if (!qw || !sw || !smooth_down || (M > 0 && (!qx || !sx || !qx_down || !sx_down)))
        return SVDQ_ERR_INVALID_ARGUMENT;
    if (rank > 0 && (!l2t || (M > 0 && !T))) return SVDQ_ERR_INVALID_ARGUMENT;
    const size_t ws = svdq_mlp_workspace_bytes(M, N, rank_down);
    if (rank_down > 0 && (!l1t_down || (M > 0 && (!T_down || !workspace || workspace_bytes < ws))))
        return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(qx) || !aligned16(sx) || !aligned16(T) || !aligned16(qw) || !aligned16(sw) ||
        !aligned16(l2t) || !aligned16(bias) || !aligned16(smooth_down) || !aligned16(l1t_down) ||
        !aligned16(qx_down) || !aligned16(sx_down) || !aligned16(T_down) || !aligned16(Y_up) ||
        !aligned16(workspace))
        return SVDQ_ERR_MISALIGNED;
    {
        const int64_t rb = (int64_t)svdq_qrow_bytes(K, SVDQ_QFMT_FP6);
        if (!fits_buffer(M, rb) || !fits_buffer(N, rb) || !fits_buffer(K / SVDQ_GROUP, 4LL * M) ||
            !fits_buffer(K / SVDQ_GROUP, 4LL * N) || !fits_buffer(M, (int64_t)svdq_qrow_bytes(N, SVDQ_QFMT_FP6)))
            return SVDQ_ERR_UNSUPPORTED_SHAPE;
    }
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    svdq::MlpOut out{smooth_down, rank_down ? l1t_down : nullptr, rank_down, qx_down, sx_down,
                     rank_down ? static_cast<float *>(workspace) : nullptr, Y_up};
    st = launched(svdq::launch_w4a4_fp6_mlp(qx, sx, rank ? T : nullptr, qw, sw, rank ? l2t : nullptr, bias, M, N,
                                            K, rank, out, (hipStream_t)stream));
    if (st != SVDQ_OK || rank_down == 0) return st;
    return launched(svdq::launch_tpart_reduce(static_cast<const float *>(workspace), svdq::mlp_tiles_n(N), M,
                                              rank_down, T_down, (hipStream_t)stream));
}

svdq_status svdq_debug_gelu_bf16(const uint16_t *y, uint16_t *g, int n, void *stream) {
    if (n < 0 || (n > 0 && (!y || !g))) return SVDQ_ERR_INVALID_ARGUMENT;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    return launched(svdq::launch_gelu_bf16(y, g, n, (hipStream_t)stream));
}

int64_t svdq_debug_mfma_ops(int kind, int blocks, int iters) {
    if (kind < 0 || kind > 2 || blocks <= 0 || iters <= 0) return 0;
    return svdq::mfma_rate_ops_per_wave_round(kind) * (int64_t)blocks * 4 * (int64_t)iters;
}

svdq_status svdq_debug_mfma_rate(int kind, int blocks, int iters, uint64_t *out, void *stream) {
    if (kind < 0 || kind > 2 || blocks <= 0 || blocks > (1 << 20) || iters <= 0 || !out)
        return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(out)) return SVDQ_ERR_MISALIGNED;
    const svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    return launched(svdq::launch_mfma_rate(kind, blocks, iters, out, (hipStream_t)stream));
}

svdq_status svdq_w4a4_linear(const uint8_t *qx, const float *sx,
                             const uint16_t *T, const uint8_t *qw,
                             const float *sw, const uint16_t *l2t,
                             const uint16_t *bias, int M, int N, int K,
                             int rank, int group, int qfmt, void *Y,
                             int y_dtype, void *stream) {
    svdq_status st = check_w4a4_shape(M, K, rank, group);
    if (st != SVDQ_OK) return st;
    if (qfmt != SVDQ_QFMT_INT4 && qfmt != SVDQ_QFMT_FP6) return SVDQ_ERR_INVALID_ARGUMENT;
    if (N <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (y_dtype != SVDQ_BF16 && y_dtype != SVDQ_F32) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!qw || !sw || (M > 0 && (!qx || !sx || !Y))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (rank > 0 && (!l2t || (M > 0 && !T))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(qx) || !aligned16(sx) || !aligned16(T) || !aligned16(qw) ||
        !aligned16(sw) || !aligned16(l2t) || !aligned16(bias) || !aligned16(Y))
        return SVDQ_ERR_MISALIGNED;
    {
        const int64_t rb = (int64_t)svdq_qrow_bytes(K, qfmt);
        if (!fits_buffer(M, rb) || !fits_buffer(N, rb) || !fits_buffer(K / SVDQ_GROUP, 4LL * M) ||
            !fits_buffer(K / SVDQ_GROUP, 4LL * N))
            return SVDQ_ERR_UNSUPPORTED_SHAPE;
    }
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    if (qfmt == SVDQ_QFMT_FP6)
        return launched(svdq::launch_w4a4_fp6_linear(qx, sx, rank ? T : nullptr, qw, sw,
                                                     rank ? l2t : nullptr, bias, M, N, K, rank, Y,
                                                     y_dtype == SVDQ_F32, (hipStream_t)stream));
    return launched(svdq::launch_w4a4_linear(qx, sx, rank ? T : nullptr, qw, sw, rank ? l2t : nullptr,
                                             bias, M, N, K, rank, Y, y_dtype == SVDQ_F32,
                                             (hipStream_t)stream));
}

size_t w8a8_workspace_bytes(int M, int K) {
    if (M < 0 || K <= 0) return 0;
    return svdq::w8a8_workspace_size(M, K);
}

svdq_status w8a8_linear(const uint16_t *X, const int8_t *qw, float sw,
                        const uint16_t *bias, int M, int N, int K,
                        void *workspace, size_t workspace_bytes, uint16_t *Y,
                        void *stream) {
    if (M < 0 || N <= 0 || K <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K % 64 || N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if ((int64_t)K * 127 * 127 >= ((int64_t)1 << 31)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!fits_buffer(M, K) || !fits_buffer(N, K)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!std::isfinite(sw) || sw < 0.0f) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!qw || (M > 0 && (!X || !Y || !workspace))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (M > 0 && workspace_bytes < svdq::w8a8_workspace_size(M, K)) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(X) || !aligned16(qw) || !aligned16(bias) || !aligned16(workspace) || !aligned16(Y))
        return SVDQ_ERR_MISALIGNED;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    return launched(svdq::launch_w8a8_linear(X, qw, sw, bias, M, N, K, workspace, Y, (hipStream_t)stream));
}

svdq_status w4a16_linear(const uint16_t *X, const uint8_t *packed, const uint16_t *bias, int M,
                         int N, int K, int group, uint16_t *Y, void *stream) {
    if (M < 0 || N <= 0 || K <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    // a block keeps at least one row of X and its group sums in LDS
    if (group != SVDQ_GROUP || K % SVDQ_GROUP || svdq::w4a16_rows_per_block(1, K) < 1)
        return SVDQ_ERR_UNSUPPORTED_SHAPE;
    // X and the weight container are read through 32-bit buffer offsets;
    // blocks are numbered in one grid dimension
    if (!fits_buffer(M, 2LL * K) || !fits_buffer(1, (int64_t)svdq::w4a16_container_bytes(K, N)) ||
        2 * (((int64_t)N + 31) / 32) * (int64_t)M >= ((int64_t)1 << 31))
        return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!packed || (M > 0 && (!X || !Y))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(X) || !aligned16(packed) || !aligned16(bias) || !aligned16(Y)) return SVDQ_ERR_MISALIGNED;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    return launched(svdq::launch_w4a16_linear(X, packed, bias, M, N, K, Y, (hipStream_t)stream));
}

svdq_status svdq_mx_quantize_act(const uint16_t *X, const float *smooth, const uint16_t *l1t, int M,
                                 int K, int rank, uint8_t *qx, uint8_t *ux, uint16_t *T, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    svdq_status st = check_w4a4_shape(M, K, rank, SVDQ_GROUP);
    if (st != SVDQ_OK) return st;
    if (!smooth || (M > 0 && (!X || !qx || !ux))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (rank > 0 && (!l1t || (M > 0 && !T))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (workspace && workspace_bytes < svdq::act_workspace_size(M, K, rank)) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(X) || !aligned16(smooth) || !aligned16(l1t) || !aligned16(qx) || !aligned16(ux) ||
        !aligned16(T) || !aligned16(workspace))
        return SVDQ_ERR_MISALIGNED;
    if (!fits_buffer(M, K / 2) || !fits_buffer(K / 32, (int64_t)svdq::mx_scale_ld(M)))
        return SVDQ_ERR_UNSUPPORTED_SHAPE;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    return launched(svdq::launch_mx_quantize_act(X, smooth, rank ? l1t : nullptr, M, K, rank, qx, ux,
                                                 rank ? T : nullptr, static_cast<float *>(workspace),
                                                 (hipStream_t)stream));
}

svdq_status svdq_mx_linear(const uint8_t *qx, const uint8_t *ux, const uint16_t *T, const uint8_t *qw,
                           const uint8_t *uw, const uint16_t *l2t, const uint16_t *bias, int M, int N, int K,
                           int rank, void *Y, int y_dtype, void *stream) {
    svdq_status st = check_w4a4_shape(M, K, rank, SVDQ_GROUP);
    if (st != SVDQ_OK) return st;
    if (N <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (y_dtype != SVDQ_BF16 && y_dtype != SVDQ_F32) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!qw || !uw || (M > 0 && (!qx || !ux || !Y))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (rank > 0 && (!l2t || (M > 0 && !T))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(qx) || !aligned16(ux) || !aligned16(T) || !aligned16(qw) || !aligned16(uw) ||
        !aligned16(l2t) || !aligned16(bias) || !aligned16(Y))
        return SVDQ_ERR_MISALIGNED;
    if (!fits_buffer(M, K / 2) || !fits_buffer(N, K / 2) || !fits_buffer(K / 32, (int64_t)svdq::mx_scale_ld(M)) ||
        !fits_buffer(K / 32, (int64_t)svdq::mx_scale_ld(N)))
        return SVDQ_ERR_UNSUPPORTED_SHAPE;
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    return launched(svdq::launch_mx_linear(qx, ux, rank ? T : nullptr, qw, uw, rank ? l2t : nullptr, bias, M, N,
                                           K, rank, Y, y_dtype == SVDQ_F32, (hipStream_t)stream));
}

svdq_status svdq_debug_group_partials(const uint8_t *qx, const uint8_t *qw,
                                      int M, int N, int K, int group, int qfmt,
                                      int32_t *P, void *stream) {
    svdq_status st = check_w4a4_shape(M, K, 0, group);
    if (st != SVDQ_OK) return st;
    if (qfmt != SVDQ_QFMT_INT4 && qfmt != SVDQ_QFMT_FP6) return SVDQ_ERR_INVALID_ARGUMENT;
    if (N <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!qw || (M > 0 && (!qx || !P))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(qx) || !aligned16(qw) || !aligned16(P)) return SVDQ_ERR_MISALIGNED;
    {
        const int64_t rb = (int64_t)svdq_qrow_bytes(K, qfmt);
        if (!fits_buffer(M, rb) || !fits_buffer(N, rb)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    }
    st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    if (qfmt == SVDQ_QFMT_FP6)
        return launched(svdq::launch_w4a4_fp6_partials(qx, qw, M, N, K, P, (hipStream_t)stream));
    return launched(svdq::launch_w4a4_partials(qx, qw, M, N, K, P, (hipStream_t)stream));
}

svdq_status w8a8_debug_acc(const int8_t *qx, const int8_t *qw, int M, int N,
                           int K, int32_t *acc, void *stream) {
    if (M < 0 || N <= 0 || K <= 0) return SVDQ_ERR_INVALID_ARGUMENT;
    if (K % 64 || N % 8) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!fits_buffer(M, K) || !fits_buffer(N, K)) return SVDQ_ERR_UNSUPPORTED_SHAPE;
    if (!qw || (M > 0 && (!qx || !acc))) return SVDQ_ERR_INVALID_ARGUMENT;
    if (!aligned16(qx) || !aligned16(qw) || !aligned16(acc)) return SVDQ_ERR_MISALIGNED;
    svdq_status st = current_device_ok();
    if (st != SVDQ_OK) return st;
    if (M == 0) return SVDQ_OK;
    return launched(svdq::launch_w8a8_acc(qx, qw, M, N, K, acc, (hipStream_t)stream));
}

}  // extern "C"
