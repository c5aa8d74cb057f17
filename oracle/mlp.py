"""Oracle for the MLP pair on the device: the up-projection's output goes
through GELU and straight into the down-projection's activation quantizer.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

[HF-SVDQ] method paragraph (4-bit weights and activations, 16-bit low-rank
branch) and "Nunchaku Lite" paragraph (svdq_w4a4 on the MLP projections,
fused kernels): a DiT MLP is up-projection, GELU, down-projection, both
projections svdq_w4a4 linears. Fusing the pair means the down-projection's
input, GELU(y_up), is never written: the up-projection's epilogue emits the
down-projection's INT4 codes, group scales and low-rank T directly. The pages
say nothing about the GELU. Readings:

  G1  GELU is the exact erf form, GELU(y) = y Phi(y) = (y / 2) erfc(-y / sqrt 2),
      of the up-projection's bf16 output, rounded once to bf16 (nearest even):
      the down-projection takes 16-bit activations, and one rounding of the
      exact value is the only form with a single right answer;
  G2  the down-projection's activation side is the plain svdq_w4a4 one on
      g = GELU(y_up): X_hat = RN32(g / s_down), group-64 INT4 codes and scales,
      T_down = bf16(g L1s_down) (readings R6-R13 of ``oracle/svdquant.py``);
  G3  y_up itself is the up-projection's bf16 output (reading R12).

Parity status: ``gelu_bf16`` is pinned by tests/test_oracle_mlp.py against an
independent evaluation of erf to 200 significant digits (Python's decimal
module, power series, pi by Machin's formula) with exact rational rounding,
closed-form tail bounds for |y| >= 16, and planted mistakes (the tanh
approximation; 1 + erf evaluated with cancellation). The rest composes
functions of ``oracle/svdquant.py`` pinned there.
"""

from __future__ import annotations

import numpy as np
from scipy.special import erfc

from . import svdquant as sq

F64 = np.float64
# relative error bound of the float64 evaluation below (erfc to a few ulps,
# the argument's rounding amplified by 2 z^2 <= 256 for |y| < 16, two
# products): far above what it is, far below bf16's half-ulp of 2^-9
EVAL_REL_ERR = 1e-12


def gelu_exact64(y):
    """GELU(y) = (y / 2) erfc(-y / sqrt 2) in float64 (reading G1): the erfc
    form has no cancellation for negative y, where 1 + erf(y / sqrt 2) would
    lose every digit."""
    y = np.asarray(y, dtype=F64)
    with np.errstate(invalid="ignore", over="ignore"):
        return 0.5 * y * erfc(-y / np.sqrt(2.0))


def gelu_bf16(y):
    """bf16(GELU(y)) with one rounding of the exact value (reading G1).

    The float64 value is within EVAL_REL_ERR of the exact one; when that
    interval holds a bf16 rounding boundary the result is decided from what
    is known exactly: GELU(y) > y / 2 for every y != 0 (the excess
    (y / 2) erf(y / sqrt 2) is positive), which settles the only such case,
    tiny |y| whose y / 2 is a tie of the subnormal grid. Any other ambiguity
    raises."""
    y = np.asarray(y, dtype=F64)
    g = gelu_exact64(y)
    lo = sq.bf16_round(g - np.abs(g) * EVAL_REL_ERR)
    hi = sq.bf16_round(g + np.abs(g) * EVAL_REL_ERR)
    out = sq.bf16_round(g)
    amb = np.isfinite(g) & (lo != hi)
    if np.any(amb):
        tiny = amb & (np.abs(y) < 2.0 ** -120)
        if np.any(amb & ~tiny):
            raise ArithmeticError("GELU rounding not decided by the float64 evaluation")
        # g sits on a tie at y / 2 up to its error; the exact value is larger
        out = np.where(tiny, hi, out)
    return out


def down_activation_side(y_up, prep_down):
    """What the fused epilogue emits for the down-projection (reading G2):
    g = GELU(y_up) (bf16), its INT4 codes qx [M, N_up], group scales sx
    [N_up / 64, M] and T = bf16(g L1s_down)."""
    g = gelu_bf16(y_up)
    qx, sx = sq.quantize_activations(g, prep_down["s"])
    T = sq.lowrank_down(g, prep_down["L1s"])
    return {"g": g, "qx": qx, "sx": sx, "T": T}


def forward(X, prep_up, bias_up, prep_down, bias_down, out="bf16"):
    """The whole pair: y_up = svdq linear (bf16), g = GELU(y_up), y_down = svdq
    linear of g."""
    up = sq.forward(X, prep_up, bias_up, "bf16")
    side = down_activation_side(up["y"], prep_down)
    down = sq.forward(side["g"], prep_down, bias_down, out)
    return {"y_up": up["y"], **side, "y_down": down["y"], "y_down64": down["y64"]}
