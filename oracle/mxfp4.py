"""Oracle for the MXFP4 variant of the SVDQuant W4A4 linear.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

[HF-SVDQ] "Nunchaku Lite" paragraph: svdq_w4a4 layers come in an INT4 and an
NVFP4 variant; the hardware paragraph: the 4-bit float variant needs a GPU
with native 4-bit float matrix units, older ones use INT4. The pages say no
more about the float format. Readings:
  F0  on gfx950 the native 4-bit float format is OCP MXFP4 (FP4 E2M1
      elements with one power-of-two E8M0 scale per block of 32 along K,
      applied by the scaled MFMA itself); NVFP4's E4M3 block-16 scales have
      no native path there, so the variant is built as MXFP4 (the OCP
      Microscaling Formats v1.0 definitions below, not on the pages);
  F1  everything outside the 4-bit product is the INT4 variant's:
      smoothing, the 16-bit low-rank branch, the residual R = diag(s)(W -
      L1s L2) on the stored factors, T = bf16(X L1s), bias, one rounding of
      y (readings R1-R5, R12 of ``oracle/svdquant.py``);
  F2  block of 32 consecutive values along K (a row of X_hat or a column of
      R): amax = max |v|; shared exponent e = floor(log2 amax) - 2 (2 = the
      exponent of E2M1's largest value 6 = 1.5 * 2^2), clamped to
      [-127, 127]; an all-zero block takes e = -127; scale 2^e stored as the
      E8M0 byte e + 127;
  F3  element code = E2M1 of v / 2^e (exact: a power of two) rounded to
      nearest, ties to the even mantissa, magnitudes above 6 saturate to 6;
      a value that rounds to zero is +0 (code 0);
  F4  E2M1 code: bit 3 sign, bits 2-1 exponent, bit 0 mantissa; magnitudes
      0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7;
  F5  y = sum_b 2^(ex_b + ew_b) sum_{k in b} e2m1(qx_k) e2m1(qw_k) + T L2 +
      bias, in float64 (every product is exact there) and rounded once.

Parity status: pinned by tests/test_oracle_mxfp4.py (the E2M1 rounding table
derived by hand, brute force in exact rational arithmetic, power-of-two
scaling invariance, on-grid exactness, idempotent requantization, planted
mistakes).
"""

from __future__ import annotations

import numpy as np

from . import svdquant as sq

BLOCK = 32
EMAX_ELEM = 2
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
F64 = np.float64


def e2m1_round(q):
    """Magnitude-and-sign rounding of values to the E2M1 grid (reading F3):
    round to nearest with ties to the even mantissa, saturate at 6.
    Returns float64 values on the grid (zero as +0)."""
    q = np.asarray(q, dtype=F64)
    m = np.abs(q)
    # quantum 0.5 below 2, 1 in [2, 4), 2 from 4 on; np.rint is
    # half-to-even, and in each binade the even multiple of the quantum is the
    # even mantissa
    r = np.where(m < 2.0, np.rint(2.0 * m) / 2.0,
                 np.where(m < 4.0, np.rint(m), 2.0 * np.rint(m / 2.0)))
    r = np.minimum(r, 6.0)
    out = np.where(q < 0, -r, r)
    return np.where(out == 0, 0.0, out)


def e2m1_encode(v):
    """Grid values -> 4-bit codes (reading F4)."""
    v = np.asarray(v, dtype=F64)
    m = np.abs(v)
    mag = np.searchsorted(E2M1_MAG, m)
    if not np.all(E2M1_MAG[np.minimum(mag, 7)] == m):
        raise ValueError("value not on the E2M1 grid")
    return (mag + np.where(v < 0, 8, 0)).astype(np.uint8)


def e2m1_decode(codes):
    c = np.asarray(codes, dtype=np.int64)
    mag = E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def shared_exponent(amax):
    """e = floor(log2 amax) - 2 clamped to [-127, 127]; amax == 0 -> -127
    (reading F2). frexp gives amax = f 2^x with f in [0.5, 1), so
    floor(log2 amax) = x - 1 exactly."""
    amax = np.asarray(amax, dtype=F64)
    _, x = np.frexp(amax)
    e = np.where(amax > 0, x - 1 - EMAX_ELEM, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_rows(V, block=BLOCK):
    """MXFP4 of each row of V [rows, K] in blocks of `block` along K.
    Returns (codes uint8 [rows, K], exponents int64 [rows, K / block])."""
    V = np.asarray(V, dtype=F64)
    rows, K = V.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    Vb = V.reshape(rows, K // block, block)
    e = shared_exponent(np.max(np.abs(Vb), axis=2) if rows else np.zeros((0, K // block)))
    q = e2m1_round(Vb / np.ldexp(1.0, e)[:, :, None])
    return e2m1_encode(q).reshape(rows, K), e


def dequantize_rows(codes, e, block=BLOCK):
    """codes [rows, K], exponents [rows, K / block] -> float64 values."""
    v = e2m1_decode(codes)
    return v * np.repeat(np.ldexp(1.0, np.asarray(e)), block, axis=1)


def quantize_activations(X, s, block=BLOCK):
    """X_hat = RN32(X / s), then MXFP4 per row (readings F1, F2)."""
    Xh = sq.smooth_activations(X, s).astype(F64)
    return quantize_rows(Xh, block)


def prepare_from_factors(W, s, L1s, L2, block=BLOCK):
    """Residual R32 = RN32(s (W - L1s L2)) as in the INT4 variant, its columns
    quantized to MXFP4 along K: qw [N, K] codes (one row per output column),
    ew [N, K/32] exponents."""
    R32 = sq.residual(W, s, L1s, L2)
    qw, ew = quantize_rows(np.asarray(R32, dtype=F64).T, block)
    return {"s": sq.rn32(s), "L1s": np.asarray(L1s, dtype=F64), "L2": np.asarray(L2, dtype=F64),
            "R32": R32, "qw": qw, "ew": ew}


def prepare_weights(W, act_absmax, rank, alpha=sq.ALPHA, block=BLOCK):
    """Smoothing and low-rank factors as in the INT4 variant, then
    prepare_from_factors."""
    s = sq.smoothing_factors(act_absmax, W, alpha)
    L1s, L2, _ = sq.lowrank_factors(W, s, rank)
    return prepare_from_factors(W, s, L1s, L2, block)


def forward(X, prep, bias=None, out="bf16", block=BLOCK):
    """The MXFP4 linear on prepared weights (reading F5). Returns qx, ex, T,
    y64 (float64, before rounding) and y (rounded to bf16 or fp32)."""
    qx, ex = quantize_activations(X, prep["s"], block)
    main = dequantize_rows(qx, ex, block) @ dequantize_rows(prep["qw"], prep["ew"], block).T
    T = sq.lowrank_down(X, prep["L1s"])
    y64 = main + np.asarray(T, dtype=F64) @ np.asarray(prep["L2"], dtype=F64)
    if bias is not None:
        y64 = y64 + np.asarray(bias, dtype=F64)[None, :]
    y = sq.rn32(y64).astype(F64) if out == "f32" else sq.bf16_round(y64)
    return {"qx": qx, "ex": ex, "T": T, "y64": y64, "y": y}
