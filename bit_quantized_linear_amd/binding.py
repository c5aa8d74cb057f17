"""ctypes binding of libsvdq.so (interface: include/svdq.h).

Argument marshalling only: host entry points take numpy arrays, device entry
points take torch tensors resident on the GPU (their data pointers are passed
through) and the current torch stream. Nothing here computes any step of the
linear; if the library is missing every call raises.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsvdq.so")

SVDQ_OK = 0
SVDQ_ERR_INVALID_ARGUMENT = 1
SVDQ_ERR_UNSUPPORTED_SHAPE = 2
SVDQ_ERR_UNSUPPORTED_DEVICE = 3
SVDQ_ERR_MISALIGNED = 4
SVDQ_ERR_NUMERICAL = 5
SVDQ_ERR_HIP = 6
SVDQ_BF16 = 0
SVDQ_F32 = 1
QFMT_INT4 = 0
QFMT_FP6 = 1
GROUP = 64

_vp, _i, _f, _sz = C.c_void_p, C.c_int, C.c_float, C.c_size_t

# name -> (restype, argtypes), mirroring include/svdq.h
SIGNATURES = {
    "svdq_status_string": (C.c_char_p, [_i]),
    "svdq_version": (_i, []),
    "svdq_qrow_bytes": (_sz, [_i, _i]),
    "svdq_repack_codes": (_i, [_vp, _i, _i, _i, _vp]),
    "svdq_check_device": (_i, [_i]),
    "svdq_prepare_weights": (_i, [_vp, _i, _i, _vp, _f, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "svdq_prepare_residual": (_i, [_vp, _i, _i, _vp, _vp, _vp, _i, _i, _vp, _vp]),
    "w8a8_prepare_weights": (_i, [_vp, _i, _i, _vp, _vp]),
    "svdq_channel_absmax": (_i, [_vp, _i, _i, _vp, _vp]),
    "svdq_act_workspace_bytes": (_sz, [_i, _i, _i]),
    "svdq_quantize_act": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "svdq_quantize_act_noalloc": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp]),
    "svdq_w4a4_linear": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _i, _vp]),
    "svdq_mlp_workspace_bytes": (_sz, [_i, _i, _i]),
    "svdq_w4a4_linear_gelu_quantize": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _i,
                                           _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "svdq_debug_gelu_bf16": (_i, [_vp, _vp, _i, _vp]),
    "w8a8_workspace_bytes": (_sz, [_i, _i]),
    "w8a8_linear": (_i, [_vp, _vp, _f, _vp, _i, _i, _i, _vp, _sz, _vp, _vp]),
    "svdq_mx_scale_ld": (_sz, [_i]),
    "svdq_mx_prepare_residual": (_i, [_vp, _i, _i, _vp, _vp, _vp, _i, _vp, _vp]),
    "svdq_mx_quantize_act": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "svdq_mx_linear": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _i, _vp]),
    "w4a16_weight_bytes": (_sz, [_i, _i]),
    "w4a16_prepare_weights": (_i, [_vp, _i, _i, _i, _vp]),
    "w4a16_linear": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _vp]),
    "svdq_debug_group_partials": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _vp, _vp]),
    "w8a8_debug_acc": (_i, [_vp, _vp, _i, _i, _i, _vp, _vp]),
    "svdq_debug_set_arch_override": (_i, [C.c_char_p]),
    "svdq_debug_mfma_ops": (C.c_int64, [_i, _i, _i]),
    "svdq_debug_mfma_rate": (_i, [_i, _i, _i, _vp, _vp]),
}

_lib = None


class SvdqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def lib():
    """The loaded library; raises if it was not built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_linear_amd.build` (there is no CPU fallback)")
        # one HIP runtime per process: torch (the device memory and stream
        # plumbing) is loaded first, so that this library binds to the HIP
        # runtime torch already uses instead of loading a second one beside it
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().svdq_status_string(status).decode()


def _check(fn, status):
    if status != SVDQ_OK:
        raise SvdqError(fn, status)


def _np_ptr(a, dtype):
    if a is None:
        return None
    if a.dtype != np.dtype(dtype) or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"expected a C-contiguous {np.dtype(dtype)} array")
    return a.ctypes.data


def _current_device():
    import torch

    return torch.cuda.current_device()


def _dev_ptr(t, itemsize=None, nbytes=0, name="tensor", device=None):
    """Device pointer of a torch tensor (None -> NULL).

    The library receives raw pointers and sizes, so the extent a call will
    touch is checked here, before anything is launched: the tensor must be a
    contiguous GPU tensor on the current device (`device`, looked up when not
    given) holding at least `nbytes` bytes. A violation raises TypeError
    (kind, layout, element size, device) or ValueError (too small)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError(f"{name}: device entry points take GPU tensors")
    if not t.is_contiguous():
        raise TypeError(f"{name}: tensors must be contiguous")
    if itemsize is not None and t.element_size() != itemsize:
        raise TypeError(f"{name}: expected {itemsize}-byte elements, got {t.element_size()}")
    dev = _current_device() if device is None else device
    if t.device.index != dev:
        raise TypeError(f"{name} is on cuda:{t.device.index}, the current device is cuda:{dev}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, the call needs at least {nbytes}")
    return t.data_ptr()


def _shape2(t, name):
    if t is None or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D tensor")
    return int(t.shape[0]), int(t.shape[1])


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------------ info --

def svdq_version() -> int:
    return lib().svdq_version()


def svdq_qrow_bytes(K: int, qfmt: int) -> int:
    return int(lib().svdq_qrow_bytes(K, qfmt))


def svdq_check_device(device: int = 0) -> int:
    return lib().svdq_check_device(device)


def svdq_debug_set_arch_override(arch):
    return lib().svdq_debug_set_arch_override(None if arch is None else arch.encode())


# ------------------------------------------------------------------ host --

def svdq_prepare_weights(W_bits, act_absmax, rank, alpha=0.5, group=GROUP, want_sigma=False):
    """Host preparation. W_bits: uint16 [K, N] bf16 bits; act_absmax: float32 [K]."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    act_absmax = np.ascontiguousarray(act_absmax, dtype=np.float32)
    K, N = W_bits.shape
    out = {
        "s": np.empty(K, np.float32),
        "l1t": np.empty((rank, K), np.uint16),
        "l2t": np.empty((N, rank), np.uint16),
        "qw": np.empty((N, K // 2), np.uint8),
        "sw": np.empty((max(K // group, 0), N), np.float32),
        "sigma": np.empty(rank, np.float64),
    }
    st = lib().svdq_prepare_weights(
        _np_ptr(W_bits, np.uint16), K, N, _np_ptr(act_absmax, np.float32), float(alpha), rank, group,
        out["s"].ctypes.data, out["l1t"].ctypes.data if rank else None,
        out["l2t"].ctypes.data if rank else None, out["qw"].ctypes.data, out["sw"].ctypes.data,
        out["sigma"].ctypes.data if rank else None)
    _check("svdq_prepare_weights", st)
    if not want_sigma:
        out.pop("sigma")
    return out


def svdq_prepare_residual(W_bits, smooth, l1t, l2t, group=GROUP):
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    smooth = np.ascontiguousarray(smooth, dtype=np.float32)
    l1t = np.ascontiguousarray(l1t, dtype=np.uint16)
    l2t = np.ascontiguousarray(l2t, dtype=np.uint16)
    K, N = W_bits.shape
    rank = l1t.shape[0]
    qw = np.empty((N, K // 2), np.uint8)
    sw = np.empty((K // group, N), np.float32)
    st = lib().svdq_prepare_residual(_np_ptr(W_bits, np.uint16), K, N, _np_ptr(smooth, np.float32),
                                     l1t.ctypes.data if rank else None, l2t.ctypes.data if rank else None,
                                     rank, group, qw.ctypes.data, sw.ctypes.data)
    _check("svdq_prepare_residual", st)
    return {"qw": qw, "sw": sw}


def svdq_repack_codes(q, K, qfmt):
    """Canonical INT4 rows [rows, K/2] -> container `qfmt` rows."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows = q.shape[0]
    out = np.empty((rows, svdq_qrow_bytes(K, qfmt)), np.uint8)
    st = lib().svdq_repack_codes(q.ctypes.data if rows else None, rows, K, qfmt,
                                 out.ctypes.data if rows else None)
    _check("svdq_repack_codes", st)
    return out


def w8a8_prepare_weights(W_bits):
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    K, N = W_bits.shape
    qw = np.empty((N, K), np.int8)
    sw = np.zeros(1, np.float32)
    st = lib().w8a8_prepare_weights(_np_ptr(W_bits, np.uint16), K, N, qw.ctypes.data, sw.ctypes.data)
    _check("w8a8_prepare_weights", st)
    return qw, float(sw[0])


def svdq_mx_scale_ld(rows) -> int:
    """Row stride (bytes) of an MXFP4 scale matrix [K/32, ld] for `rows` rows."""
    return int(lib().svdq_mx_scale_ld(rows))


def svdq_mx_prepare_residual(W_bits, smooth, l1t, l2t):
    """MXFP4 residual of a bf16 weight W [K, N] given smoothing and factors:
    codes (MX container, N rows of K/2 bytes) and E8M0 scales [K/32, ld(N)]."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    smooth = np.ascontiguousarray(smooth, dtype=np.float32)
    l1t = np.ascontiguousarray(l1t, dtype=np.uint16)
    l2t = np.ascontiguousarray(l2t, dtype=np.uint16)
    K, N = W_bits.shape
    rank = l1t.shape[0]
    qw = np.empty((N, K // 2), np.uint8)
    uw = np.zeros((max(K // 32, 0), svdq_mx_scale_ld(N)), np.uint8)
    st = lib().svdq_mx_prepare_residual(_np_ptr(W_bits, np.uint16), K, N, _np_ptr(smooth, np.float32),
                                        l1t.ctypes.data if rank else None, l2t.ctypes.data if rank else None,
                                        rank, qw.ctypes.data, uw.ctypes.data)
    _check("svdq_mx_prepare_residual", st)
    return {"qw": qw, "uw": uw}


def w4a16_weight_bytes(K, N) -> int:
    return int(lib().w4a16_weight_bytes(K, N))


def w4a16_prepare_weights(W_bits, group=GROUP):
    """W4A16 weight container (uint8, w4a16_weight_bytes(K, N) bytes) of a
    bf16 weight W [K, N]."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    K, N = W_bits.shape
    nbytes = w4a16_weight_bytes(K, N)
    out = np.empty(max(nbytes, 1), np.uint8)
    st = lib().w4a16_prepare_weights(_np_ptr(W_bits, np.uint16), K, N, group, out.ctypes.data)
    _check("w4a16_prepare_weights", st)
    return out[:nbytes]


# ---------------------------------------------------------------- device --
#
# Every wrapper checks, before calling into the library, that each tensor
# covers the extent the call will read or write for the sizes it passes (the
# library sees only pointers and sizes), and that each tensor is on the
# current device.

def svdq_channel_absmax(X, absmax, stream=None):
    M, K = _shape2(X, "X")
    dev = _current_device()
    st = lib().svdq_channel_absmax(_dev_ptr(X, 2, M * K * 2, "X", dev), M, K,
                                   _dev_ptr(absmax, 4, K * 4, "absmax", dev), _stream(stream))
    _check("svdq_channel_absmax", st)


def svdq_act_workspace_bytes(M, K, rank) -> int:
    return int(lib().svdq_act_workspace_bytes(M, K, rank))


def _ws(workspace, dev):
    if workspace is None:
        return None, 0
    return _dev_ptr(workspace, None, 0, "workspace", dev), workspace.numel() * workspace.element_size()


def svdq_quantize_act(X, smooth, l1t, qx, sx, T, rank, group=GROUP, qfmt=QFMT_INT4, workspace=None,
                      stream=None):
    M, K = _shape2(X, "X")
    dev = _current_device()
    G = K // group if group > 0 else 0
    wp, wb = _ws(workspace, dev)
    st = lib().svdq_quantize_act(
        _dev_ptr(X, 2, M * K * 2, "X", dev), _dev_ptr(smooth, 4, K * 4, "smooth", dev),
        _dev_ptr(l1t, 2, rank * K * 2, "l1t", dev), M, K, rank, group, qfmt,
        _dev_ptr(qx, 1, M * svdq_qrow_bytes(K, qfmt), "qx", dev), _dev_ptr(sx, 4, G * M * 4, "sx", dev),
        _dev_ptr(T, 2, M * rank * 2, "T", dev), wp, wb, _stream(stream))
    _check("svdq_quantize_act", st)


def svdq_quantize_act_noalloc(X, smooth, l1t, qx, sx, T, rank, group=GROUP, qfmt=QFMT_INT4, stream=None):
    """svdq_quantize_act with the library's fixed device scratch instead of a
    caller workspace (allocates nothing)."""
    M, K = _shape2(X, "X")
    dev = _current_device()
    G = K // group if group > 0 else 0
    st = lib().svdq_quantize_act_noalloc(
        _dev_ptr(X, 2, M * K * 2, "X", dev), _dev_ptr(smooth, 4, K * 4, "smooth", dev),
        _dev_ptr(l1t, 2, rank * K * 2, "l1t", dev), M, K, rank, group, qfmt,
        _dev_ptr(qx, 1, M * svdq_qrow_bytes(K, qfmt), "qx", dev), _dev_ptr(sx, 4, G * M * 4, "sx", dev),
        _dev_ptr(T, 2, M * rank * 2, "T", dev), _stream(stream))
    _check("svdq_quantize_act_noalloc", st)


def _linear_operands(qx, sx, T, qw, sw, l2t, bias, M, N, K, rank, group, qfmt, dev):
    """Checked pointers of the W4A4 GEMM's inputs (shared by the linear and
    the fused MLP entry point)."""
    R = svdq_qrow_bytes(K, qfmt)
    G = K // group if group > 0 else 0
    return (_dev_ptr(qx, 1, M * R, "qx", dev), _dev_ptr(sx, 4, G * M * 4, "sx", dev),
            _dev_ptr(T, 2, M * rank * 2, "T", dev), _dev_ptr(qw, 1, N * R, "qw", dev),
            _dev_ptr(sw, 4, G * N * 4, "sw", dev), _dev_ptr(l2t, 2, N * rank * 2, "l2t", dev),
            _dev_ptr(bias, 2, N * 2, "bias", dev))


def svdq_w4a4_linear(qx, sx, T, qw, sw, l2t, bias, Y, M, N, K, rank, group=GROUP, qfmt=QFMT_INT4,
                     stream=None):
    dev = _current_device()
    y_dtype = SVDQ_F32 if Y.element_size() == 4 else SVDQ_BF16
    ins = _linear_operands(qx, sx, T, qw, sw, l2t, bias, M, N, K, rank, group, qfmt, dev)
    st = lib().svdq_w4a4_linear(*ins, M, N, K, rank, group, qfmt,
                                _dev_ptr(Y, None, M * N * Y.element_size(), "Y", dev), y_dtype, _stream(stream))
    _check("svdq_w4a4_linear", st)


def svdq_mlp_workspace_bytes(M, N, rank_down) -> int:
    return int(lib().svdq_mlp_workspace_bytes(M, N, rank_down))


def svdq_w4a4_linear_gelu_quantize(qx, sx, T, qw, sw, l2t, bias, M, N, K, rank, smooth_down, l1t_down,
                                   rank_down, qx_down, sx_down, T_down, Y_up=None, workspace=None,
                                   group=GROUP, stream=None):
    dev = _current_device()
    ins = _linear_operands(qx, sx, T, qw, sw, l2t, bias, M, N, K, rank, group, QFMT_FP6, dev)
    Gd = N // group if group > 0 else 0
    ws_need = svdq_mlp_workspace_bytes(M, N, rank_down)
    st = lib().svdq_w4a4_linear_gelu_quantize(
        *ins, M, N, K, rank, group, _dev_ptr(smooth_down, 4, N * 4, "smooth_down", dev),
        _dev_ptr(l1t_down, 2, rank_down * N * 2, "l1t_down", dev), rank_down,
        _dev_ptr(qx_down, 1, M * svdq_qrow_bytes(N, QFMT_FP6), "qx_down", dev),
        _dev_ptr(sx_down, 4, Gd * M * 4, "sx_down", dev), _dev_ptr(T_down, 2, M * rank_down * 2, "T_down", dev),
        _dev_ptr(Y_up, 2, M * N * 2, "Y_up", dev), _dev_ptr(workspace, None, ws_need, "workspace", dev),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check("svdq_w4a4_linear_gelu_quantize", st)


def svdq_debug_gelu_bf16(y, g, stream=None):
    dev = _current_device()
    n = y.numel()
    st = lib().svdq_debug_gelu_bf16(_dev_ptr(y, 2, n * 2, "y", dev), _dev_ptr(g, 2, n * 2, "g", dev), n,
                                    _stream(stream))
    _check("svdq_debug_gelu_bf16", st)


def w8a8_workspace_bytes(M, K) -> int:
    return int(lib().w8a8_workspace_bytes(M, K))


def w8a8_linear(X, qw, sw, bias, workspace, Y, stream=None):
    M, K = _shape2(X, "X")
    N, Kw = _shape2(qw, "qw")
    if Kw != K:
        raise ValueError(f"qw has {Kw} columns, X has K = {K}")
    dev = _current_device()
    ws_need = w8a8_workspace_bytes(M, K)
    st = lib().w8a8_linear(_dev_ptr(X, 2, M * K * 2, "X", dev), _dev_ptr(qw, 1, N * K, "qw", dev), float(sw),
                           _dev_ptr(bias, 2, N * 2, "bias", dev), M, N, K,
                           _dev_ptr(workspace, None, ws_need, "workspace", dev),
                           workspace.numel() * workspace.element_size(),
                           _dev_ptr(Y, 2, M * N * 2, "Y", dev), _stream(stream))
    _check("w8a8_linear", st)


def svdq_mx_quantize_act(X, smooth, l1t, qx, ux, T, rank, workspace=None, stream=None):
    M, K = _shape2(X, "X")
    dev = _current_device()
    wp, wb = _ws(workspace, dev)
    st = lib().svdq_mx_quantize_act(
        _dev_ptr(X, 2, M * K * 2, "X", dev), _dev_ptr(smooth, 4, K * 4, "smooth", dev),
        _dev_ptr(l1t, 2, rank * K * 2, "l1t", dev), M, K, rank, _dev_ptr(qx, 1, M * (K // 2), "qx", dev),
        _dev_ptr(ux, 1, (K // 32) * svdq_mx_scale_ld(M), "ux", dev), _dev_ptr(T, 2, M * rank * 2, "T", dev),
        wp, wb, _stream(stream))
    _check("svdq_mx_quantize_act", st)


def svdq_mx_linear(qx, ux, T, qw, uw, l2t, bias, Y, M, N, K, rank, stream=None):
    dev = _current_device()
    y_dtype = SVDQ_F32 if Y.element_size() == 4 else SVDQ_BF16
    st = lib().svdq_mx_linear(
        _dev_ptr(qx, 1, M * (K // 2), "qx", dev), _dev_ptr(ux, 1, (K // 32) * svdq_mx_scale_ld(M), "ux", dev),
        _dev_ptr(T, 2, M * rank * 2, "T", dev), _dev_ptr(qw, 1, N * (K // 2), "qw", dev),
        _dev_ptr(uw, 1, (K // 32) * svdq_mx_scale_ld(N), "uw", dev), _dev_ptr(l2t, 2, N * rank * 2, "l2t", dev),
        _dev_ptr(bias, 2, N * 2, "bias", dev), M, N, K, rank,
        _dev_ptr(Y, None, M * N * Y.element_size(), "Y", dev), y_dtype, _stream(stream))
    _check("svdq_mx_linear", st)


def w4a16_linear(X, packed, bias, Y, N, group=GROUP, stream=None):
    """Y [M, N] bf16 = X [M, K] bf16 times the W4A16 container `packed`."""
    M, K = _shape2(X, "X")
    dev = _current_device()
    st = lib().w4a16_linear(_dev_ptr(X, 2, M * K * 2, "X", dev),
                            _dev_ptr(packed, 1, w4a16_weight_bytes(K, N), "packed", dev),
                            _dev_ptr(bias, 2, N * 2, "bias", dev), M, N, K, group,
                            _dev_ptr(Y, 2, M * N * 2, "Y", dev), _stream(stream))
    _check("w4a16_linear", st)


def svdq_debug_group_partials(qx, qw, P, M, N, K, group=GROUP, qfmt=QFMT_INT4, stream=None):
    dev = _current_device()
    R = svdq_qrow_bytes(K, qfmt)
    G = K // group if group > 0 else 0
    st = lib().svdq_debug_group_partials(_dev_ptr(qx, 1, M * R, "qx", dev), _dev_ptr(qw, 1, N * R, "qw", dev),
                                         M, N, K, group, qfmt, _dev_ptr(P, 4, G * M * N * 4, "P", dev),
                                         _stream(stream))
    _check("svdq_debug_group_partials", st)


def w8a8_debug_acc(qx, qw, acc, M, N, K, stream=None):
    dev = _current_device()
    st = lib().w8a8_debug_acc(_dev_ptr(qx, 1, M * K, "qx", dev), _dev_ptr(qw, 1, N * K, "qw", dev), M, N, K,
                              _dev_ptr(acc, 4, M * N * 4, "acc", dev), _stream(stream))
    _check("w8a8_debug_acc", st)


def svdq_debug_mfma_ops(kind, blocks, iters) -> int:
    return int(lib().svdq_debug_mfma_ops(kind, blocks, iters))


def svdq_debug_mfma_rate(kind, blocks, iters, out, stream=None):
    """Back-to-back MFMAs of one kind on every SIMD; out: uint64 device tensor
    of 8 * blocks values (per wave: shader-clock span, real-time span)."""
    dev = _current_device()
    st = lib().svdq_debug_mfma_rate(kind, blocks, iters, _dev_ptr(out, 8, 8 * 8 * blocks, "out", dev),
                                    _stream(stream))
    _check("svdq_debug_mfma_rate", st)


# ------------------------------------------------ convenience allocation --

def w8a8_workspace_offset_codes() -> int:
    """Byte offset of the int8 codes of X inside the w8a8 workspace."""
    return 8192


def w8a8_workspace_offset_scale() -> int:
    """Byte offset of the fp32 activation scale inside the w8a8 workspace."""
    return 4096
