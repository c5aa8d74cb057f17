"""GPU-test helpers: oracle preparation of a case, upload, and calls through
the C-ABI binding. Inputs always flow oracle -> library, never back."""

from __future__ import annotations

import functools

import numpy as np

from bit_quantized_linear_amd import binding as b
from bit_quantized_linear_amd import workloads as wl
from oracle import svdquant as sq
from oracle import w8a8 as o8

F64 = np.float64


def torch():
    import torch as _t

    return _t


def dev(a):
    """numpy -> contiguous GPU tensor with the same bytes (uint16 travels as int16)."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


@functools.lru_cache(maxsize=8)
def prepared_case(name: str):
    """Oracle preparation of a named case (calibrated on the case's own X)."""
    case = wl.CASES[name]
    X = wl.activations(case)
    W = wl.weight(case)
    bias = wl.bias(case)
    a = sq.channel_absmax(X["values"])
    prep = sq.prepare_weights(W["values"], a, case.rank)
    return case, X, W, bias, prep, sq.to_abi(prep)


def make_problem(M, K, N, rank, seed=0, outliers=(), bias=True, zero_rows=()):
    """A small ad-hoc problem with the generators' distributions."""
    X = wl.random_bf16(seed * 10 + 1, (M, K))
    Xv = X["values"].copy()
    for ch in outliers:
        Xv[:, ch] *= 20.0
    for r in zero_rows:
        Xv[r, :] = 0.0
    Xb = wl.bf16_bits_from_f32(Xv)
    Xv = wl.f32_from_bf16_bits(Xb)
    W = wl.random_bf16(seed * 10 + 2, (K, N), 0.02)
    bvals = wl.random_bf16(seed * 10 + 3, (N,), 0.01) if bias else None
    a = sq.channel_absmax(Xv)
    prep = sq.prepare_weights(W["values"], a, rank)
    return {"X": {"bits": Xb, "values": Xv}, "W": W, "bias": bvals, "prep": prep, "abi": sq.to_abi(prep)}


FORMATS = [b.QFMT_INT4, b.QFMT_FP6]
FORMAT_IDS = ["int4", "fp6"]


def pack_codes(codes, qfmt):
    """Oracle codes [rows, K] -> the container's bytes (test-side writers)."""
    from tests.fp6_format import pack_fp6

    return sq.pack_int4(codes) if qfmt == b.QFMT_INT4 else pack_fp6(codes)


def unpack_codes(packed, K, qfmt):
    from tests.fp6_format import unpack_fp6

    return sq.unpack_int4(packed) if qfmt == b.QFMT_INT4 else unpack_fp6(packed, K)


def weights_bytes(prep, abi, qfmt):
    """The oracle's weight codes in container `qfmt` ([N, row bytes])."""
    return abi["qw"] if qfmt == b.QFMT_INT4 else pack_codes(np.asarray(prep["qw"]).T, qfmt)


def act_workspace(M, K, rank):
    """The activation pass's optional workspace (None when it needs none)."""
    t = torch()
    n = b.svdq_act_workspace_bytes(M, K, rank)
    return t.empty(n, dtype=t.uint8, device="cuda") if n else None


def run_quantize_act(Xbits, abi, rank, qfmt=b.QFMT_INT4, split=True):
    """The activation pass as the bench runs it (with its workspace: K split
    across blocks where that fills the GPU better), or without (split=False)."""
    t = torch()
    M, K = Xbits.shape
    Xd = dev(Xbits)
    qx = t.empty((M, b.svdq_qrow_bytes(K, qfmt)), dtype=t.uint8, device="cuda")
    sx = t.empty((K // 64, M), dtype=t.float32, device="cuda")
    T = t.empty((M, max(rank, 1)), dtype=t.int16, device="cuda") if rank else None
    l1t = dev(abi["l1t"]) if rank else None
    b.svdq_quantize_act(Xd, dev(abi["s"]), l1t, qx, sx, T, rank, qfmt=qfmt,
                        workspace=act_workspace(M, K, rank) if split else None)
    t.cuda.synchronize()
    return qx, sx, T


def run_linear(qx, sx, T, abi, bias_bits, M, N, K, rank, out="bf16", qfmt=b.QFMT_INT4, qw_bytes=None):
    t = torch()
    Y = t.empty((M, N), dtype=t.float32 if out == "f32" else t.int16, device="cuda")
    qw = abi["qw"] if qw_bytes is None else qw_bytes
    b.svdq_w4a4_linear(qx, sx, T, dev(qw), dev(abi["sw"]), dev(abi["l2t"]) if rank else None,
                       dev(bias_bits) if bias_bits is not None else None, Y, M, N, K, rank, qfmt=qfmt)
    t.cuda.synchronize()
    return Y


def y_values(Y, out):
    a = host(Y)
    if out == "f32":
        return a.astype(F64)
    return sq.bf16_from_bits(a.view(np.uint16))


def w8a8_run(Xbits, qw_abi, sw, bias_bits):
    t = torch()
    M, K = Xbits.shape
    N = qw_abi.shape[0]
    ws = t.empty(b.w8a8_workspace_bytes(M, K), dtype=t.uint8, device="cuda")
    Y = t.empty((M, N), dtype=t.int16, device="cuda")
    b.w8a8_linear(dev(Xbits), dev(qw_abi), sw, dev(bias_bits) if bias_bits is not None else None, ws, Y)
    t.cuda.synchronize()
    wsh = host(ws)
    codes = wsh[b.w8a8_workspace_offset_codes(): b.w8a8_workspace_offset_codes() + M * K].view(np.int8)
    scale = wsh[b.w8a8_workspace_offset_scale(): b.w8a8_workspace_offset_scale() + 4].view(np.float32)[0]
    return Y, codes.reshape(M, K), float(scale)


def o8_prepare(Wvals):
    return o8.prepare_weights(Wvals)
