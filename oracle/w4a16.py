"""Oracle for the W4A16 linear (the awq_w4a16 layer type).

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

[HF-SVDQ] "Nunchaku Lite" paragraph: besides the svdq_w4a4 layers, the
runtime has a second layer type, awq_w4a16, with 4-bit weights and 16-bit
activations, used for the precision-sensitive normalization and modulation
layers (the adaLN modulation of FLUX, the modulation of Qwen-Image). The
pages name the layer type and its bit widths and nothing more. Readings:
  A1  the 4-bit weights use the same symmetric INT4 grid as the residual of
      the W4A4 path: per output column and group of 64 along K, scale =
      RN32(absmax / 7), code = clamp(RNE(RN32(w / scale)), -7, 7), an
      all-zero group gets scale 0 and codes 0 (readings R6-R10 of
      ``oracle/svdquant.py``), applied to W itself: no smoothing and no
      low-rank branch;
  A2  AWQ's activation-aware per-input-channel scales are chosen from
      calibration activations; at run time they are folded into the layer
      before (the normalization), so the linear itself is
      y = X dequant(Q4(W)) + bias on the bf16 X it is given; the search is
      not part of the layer;
  A3  the 16-bit activations are bf16 (the path's activation type);
  A4  y = sum_g sw[g, n] sum_{k in g} x[m, k] q[k, n] + bias[n] evaluated
      exactly (float64 here: see ``forward``) and rounded once to bf16.

Parity status: pinned by tests/test_oracle_w4a16.py (brute force in exact
rational arithmetic, on-grid weights against a plain matmul, a hand-derived
golden file, and planted mistakes that the pins must catch).
"""

from __future__ import annotations

import numpy as np

from .svdquant import GROUP, bf16_round, quantize_weights

F64 = np.float64


def prepare_weights(W, group=GROUP):
    """W [K, N] (bf16 values) -> (qw [K, N] int8 codes, sw [K/G, N] float32):
    the INT4 group quantizer of reading A1, one column at a time."""
    return quantize_weights(np.asarray(W, dtype=np.float32), group)


def dequantize(qw, sw, group=GROUP):
    """W_q[k, n] = qw[k, n] * sw[k // G, n] in float64 (exact: a 4-bit code
    times an fp32 scale)."""
    qw = np.asarray(qw, dtype=F64)
    return qw * np.repeat(np.asarray(sw, dtype=F64), group, axis=0)


def forward(X, qw, sw, bias=None, group=GROUP):
    """The W4A16 linear (reading A4). X [M, K] bf16 values, qw [K, N] codes,
    sw [K/G, N], bias [N] or None. Returns {"y64": float64 [M, N],
    "y": bf16-valued float64 [M, N]}.

    float64 holds every product x q sw exactly (8 + 3 + 24 significant bits);
    the sum over K is within a few float64 ulps of the exact value, far below
    the bf16 quantum of the result, so the single rounding to bf16 is the
    exact method's rounding except at ties no test input reaches.
    """
    X = np.asarray(X, dtype=F64)
    y64 = X @ dequantize(qw, sw, group)
    if bias is not None:
        y64 = y64 + np.asarray(bias, dtype=F64)[None, :]
    return {"y64": y64, "y": bf16_round(y64)}
