"""Oracle for the INT8 tensorwise W8A8 linear.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

[KREA-SVDQ] section "Решение: INT8 и W4A4": the first fast format is INT8
"tensorwise" -- one scale for a whole tensor -- run on the integer tensor
units. Readings taken where the pages are silent:
  W1  symmetric grid [-127, 127], scale = RN32(absmax / 127) over the whole
      tensor; the activation scale is taken per call from the X being
      multiplied (dynamic), the weight scale once at preparation (static);
  W2  code = clamp(RNE(RN32(x / scale)), -127, 127); an all-zero tensor gets
      scale 0 and codes 0;
  W3  acc = sum_k qx qw over all of K, exact (|acc| <= K 127^2 < 2^31 for the
      shapes served);
  W4  y = bf16(acc sx sw + bias), evaluated in float64 and rounded once.

Parity status: pinned by tests/test_oracle_w8a8.py (brute force on tiny
inputs, dequantize-then-matmul closed form, on-grid exactness, scaling and
sign invariants, a hand-derived golden file).
"""

from __future__ import annotations

import numpy as np

from .svdquant import bf16_round, rn32

QMAX8 = 127
F64 = np.float64


def tensor_scale(V):
    """RN32(max |V| / 127) over the whole tensor."""
    V = np.asarray(V, dtype=F64)
    amax = float(np.max(np.abs(V))) if V.size else 0.0
    return np.float32(rn32(amax / QMAX8))


def quantize_tensor(V, scale):
    """code = clamp(RNE(RN32(v / scale)), -127, 127); scale 0 -> codes 0."""
    V = np.asarray(V, dtype=F64)
    sc = float(scale)
    if sc == 0.0:
        return np.zeros(V.shape, dtype=np.int8)
    q = np.rint(rn32(V / sc).astype(F64))
    return np.clip(q, -QMAX8, QMAX8).astype(np.int8)


def prepare_weights(W):
    """W [K, N] -> (qw [K, N] int8, sw float32)."""
    sw = tensor_scale(W)
    return quantize_tensor(W, sw), sw


def quantize_activations(X):
    """X [M, K] -> (qx [M, K] int8, sx float32)."""
    sx = tensor_scale(X)
    return quantize_tensor(X, sx), sx


def accumulate(qx, qw):
    """acc = qx @ qw, exact: integer codes, |acc| < 2^31 << 2^53, so the
    float64 matmul makes no rounding. Returned as int64."""
    acc = np.asarray(qx, dtype=F64) @ np.asarray(qw, dtype=F64)
    return acc.astype(np.int64)


def forward(X, qw, sw, bias=None):
    """The W8A8 linear. Returns a dict with qx, sx, acc, y64 and y (bf16)."""
    qx, sx = quantize_activations(X)
    acc = accumulate(qx, qw)
    y64 = acc.astype(F64) * float(sx) * float(sw)
    if bias is not None:
        y64 = y64 + np.asarray(bias, dtype=F64)[None, :]
    return {"qx": qx, "sx": sx, "acc": acc, "y64": y64, "y": bf16_round(y64)}


def to_abi(qw):
    """qw [K, N] -> the library's [N, K] int8 layout (K contiguous)."""
    return np.ascontiguousarray(np.asarray(qw, dtype=np.int8).T)
