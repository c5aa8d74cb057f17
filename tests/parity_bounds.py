"""A-priori per-element error bounds for the device outputs against the
oracle (test-side helpers).

The device path computes in fp32 what the oracle computes in float64; given
the same codes and scales (checked bit-exactly first), what remains is fp32
rounding, bounded element by element here. A wrong element -- a dropped
group, a transposed scale, a missed tile -- is off by a sizeable fraction of
its own terms and fails such a bound, where a whole-matrix rel-L2 could let
a handful of them through.

W4A4 (reading R12 order: main + low-rank + bias, one output rounding):
  y32 = fl(sum_g fl(sx sw) P_g + sum_j T_j L2_j + bias) in fp32, so
  |y32 - y64| <= c u (sum_g |sx sw P_g| + sum_j |T_j L2_j| + |bias|) + c 2^-149
  + 2^-150 sum_g |P_g|
  with u = 2^-24 and c = 2 (G + r + 3) (one rounding per scale product, per
  group accumulation, per low-rank product sum, and the bias add, doubled to
  cover the matrix core's internal accumulation order; the absolute term
  covers results in fp32's subnormal range). The last term is the scale
  product fl(sx sw) rounded in fp32's subnormal range, where its error is
  absolute (at most half of 2^-149) and is multiplied by the group partial.
  The sums are bounded by Cauchy-Schwarz:
  sum_g |sx sw P_g| <= ||dequant(qx)[m]|| ||dequant(qw)[:, n]|| and
  sum_g |P_g| <= ||qx[m]|| ||qw[:, n]||.
  When the device's T differs from the oracle's (within its own checked
  bound), sum_j |dT_j| |L2_j| is added.
  The output rounding adds one unit in the last place of the output type at
  the larger of the two magnitudes (both sides round once to nearest).

W8A8: y = bf16(fl(fl(float(acc)) fl(sx sw)) + bias): four fp32 roundings of
at most |acc sx sw| + |bias|, then one bf16 ulp.
"""

from __future__ import annotations

import numpy as np

from oracle import svdquant as sq

F64 = np.float64
U32 = 2.0 ** -24
F32_TINY = 2.0 ** -149


def ulp(x, out):
    """Unit in the last place of |x| in the output type ('bf16' or 'f32'),
    with the type's subnormal quantum as the floor."""
    bits, emin = (8, -133) if out == "bf16" else (24, -149)
    a = np.maximum(np.abs(np.asarray(x, dtype=F64)), 1e-300)
    e = np.frexp(a)[1]
    return np.ldexp(1.0, np.maximum(e - bits, emin))


def w4a4_tolerance(qx, sx, qw, sw, T, L2, bias, got, ref, out, dT=None):
    """Per-element bound on |got - ref| for the W4A4 linear.

    qx [M, K] codes, sx [K/64, M], qw [K, N] codes, sw [K/64, N]; T [M, r]
    (the oracle's, float), L2 [r, N]; bias [N] or None; got / ref: the
    device's and the oracle's rounded outputs [M, N]; dT: device T minus
    oracle T [M, r], or None when the device used the oracle's T."""
    G = np.asarray(qx).shape[1] // 64
    r = 0 if T is None else np.asarray(T).shape[1]
    nx = np.linalg.norm(sq.dequantize(qx, sx), axis=1)
    nw = np.linalg.norm(sq.dequantize(np.asarray(qw).T, sw), axis=1)
    S = nx[:, None] * nw[None, :]
    if r:
        S = S + np.abs(np.asarray(T, dtype=F64)) @ np.abs(np.asarray(L2, dtype=F64))
    if bias is not None:
        S = S + np.abs(np.asarray(bias, dtype=F64))[None, :]
    c = 2.0 * (G + r + 3)
    cx = np.linalg.norm(np.asarray(qx, dtype=F64), axis=1)
    cw = np.linalg.norm(np.asarray(qw, dtype=F64), axis=0)
    tol = c * U32 * S + c * F32_TINY + 0.5 * F32_TINY * cx[:, None] * cw[None, :]
    if dT is not None and r:
        tol = tol + np.abs(np.asarray(dT, dtype=F64)) @ np.abs(np.asarray(L2, dtype=F64))
    big = np.maximum(np.abs(np.asarray(got, dtype=F64)), np.abs(np.asarray(ref, dtype=F64)))
    return tol + ulp(big, out)


def w8a8_tolerance(acc, sx, sw, bias, got, ref):
    """Per-element bound on |got - ref| for the W8A8 linear (bf16 output)."""
    S = np.abs(np.asarray(acc, dtype=F64)) * float(sx) * float(sw)
    if bias is not None:
        S = S + np.abs(np.asarray(bias, dtype=F64))[None, :]
    big = np.maximum(np.abs(np.asarray(got, dtype=F64)), np.abs(np.asarray(ref, dtype=F64)))
    return 4.0 * U32 * S + 4.0 * F32_TINY + ulp(big, "bf16")


def check_elementwise(got, ref, tol, what=""):
    got = np.asarray(got, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    bad = ~(np.abs(got - ref) <= tol)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside the bound; first "
                             f"{idx.tolist()}: got {got[bad][:5]}, ref {ref[bad][:5]}, tol {tol[bad][:5]}")
