"""Scalar brute-force tier of the oracle, for tiny inputs only.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

Pure Python, exact rational arithmetic (fractions.Fraction), one element at a
time. It takes the same definitions as ``oracle.svdquant``,
``oracle.w8a8`` and ``oracle.w4a16`` but shares none of their code and uses
a different formulation where one exists:

* fp32 rounding through ``struct`` (the C float conversion, nearest-even);
* bf16 rounding by exact rational comparison with the two neighbours;
* integer rounding by Python's ``round`` (half-to-even);
* the main product as sum_k dequant(qx[m,k]) dequant(qw[k,n]) -- one sum
  over all of K of dequantized values, with no group partials -- and the whole
  output summed exactly, then rounded once.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction


def rn32_exact(x: Fraction) -> float:
    """Correctly rounded binary32 of an exact rational (nearest-even)."""
    return _round_sig(x, 24, -149)


def bf16_exact(x: Fraction) -> float:
    """Correctly rounded bfloat16 of an exact rational (nearest-even)."""
    return _round_sig(x, 8, -133)


def _round_sig(x: Fraction, sig_bits: int, min_quantum_exp: int) -> float:
    x = Fraction(x)
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - (sig_bits - 1), min_quantum_exp)
    quantum = Fraction(2) ** qexp
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * quantum)


def div32(a: float, b: float) -> float:
    """IEEE binary32 quotient of two binary32 values."""
    return rn32_exact(Fraction(a) / Fraction(b))


def quantize_group(values, qmax):
    """Symmetric grid: scale = RN32(max|v| / qmax), code = RNE(RN32(v/scale))
    clamped to [-qmax, qmax]; an all-zero group -> scale 0, codes 0."""
    amax = max(abs(v) for v in values)
    scale = div32(amax, float(qmax))
    if scale == 0.0:
        return [0] * len(values), 0.0
    codes = []
    for v in values:
        q = round(div32(v, scale))  # Python rounds half to even
        codes.append(max(-qmax, min(qmax, q)))
    return codes, scale


def svdq_forward(X, s, L1s, L2, qw, sw, bias, group=64, out="f32"):
    """W4A4 linear on prepared weights, element by element.

    X [M][K] bf16-valued floats, s [K], L1s [K][r], L2 [r][N], qw [K][N]
    codes, sw [K/G][N], bias [N] or None. Returns (qx [M][K], sx [G][M],
    T [M][r], y [M][N]) with y rounded once to fp32 ('f32') or bf16.
    """
    M, K = len(X), len(X[0])
    N = len(qw[0])
    r = len(L2)
    G = K // group
    qx = [[0] * K for _ in range(M)]
    sx = [[0.0] * M for _ in range(G)]
    for m in range(M):
        xhat = [div32(X[m][k], s[k]) for k in range(K)]
        for g in range(G):
            codes, scale = quantize_group(xhat[g * group:(g + 1) * group], 7)
            qx[m][g * group:(g + 1) * group] = codes
            sx[g][m] = scale
    T = [[bf16_exact(sum((Fraction(X[m][k]) * Fraction(L1s[k][j]) for k in range(K)),
                         Fraction(0))) for j in range(r)] for m in range(M)]
    y = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // group
                acc += (Fraction(qx[m][k]) * Fraction(sx[g][m])) * \
                       (Fraction(qw[k][n]) * Fraction(sw[g][n]))
            for j in range(r):
                acc += Fraction(T[m][j]) * Fraction(L2[j][n])
            if bias is not None:
                acc += Fraction(bias[n])
            row.append(rn32_exact(acc) if out == "f32" else bf16_exact(acc))
        y.append(row)
    return qx, sx, T, y


def svdq_weights(W, s, L1s, L2, group=64):
    """Residual R = RN32(s (W - L1s L2)) element by element, then its INT4
    group codes per output column. Returns (qw [K][N], sw [G][N])."""
    K, N = len(W), len(W[0])
    r = len(L2)
    R = [[rn32_exact(Fraction(s[k]) * (Fraction(W[k][n]) -
                                       sum((Fraction(L1s[k][j]) * Fraction(L2[j][n])
                                            for j in range(r)), Fraction(0))))
          for n in range(N)] for k in range(K)]
    G = K // group
    qw = [[0] * N for _ in range(K)]
    sw = [[0.0] * N for _ in range(G)]
    for n in range(N):
        for g in range(G):
            codes, scale = quantize_group([R[k][n] for k in range(g * group, (g + 1) * group)], 7)
            for i, c in enumerate(codes):
                qw[g * group + i][n] = c
            sw[g][n] = scale
    return qw, sw


def smoothing(X, W, alpha=0.5):
    """s_k = RN32(a_k^alpha / w_k^(1-alpha)) for alpha = 1/2, i.e. the
    correctly rounded binary32 value of sqrt(a_k / w_k), found by exact
    rational comparison of squares against the rounding midpoints."""
    if alpha != 0.5:
        raise ValueError("brute-force smoothing supports alpha = 0.5 only")
    K = len(W)
    s = []
    for k in range(K):
        a = max(abs(X[m][k]) for m in range(len(X)))
        w = max(abs(v) for v in W[k])
        if a == 0 or w == 0:
            s.append(1.0)
            continue
        s.append(_sqrt32_exact(Fraction(a) / Fraction(w)))
    return s


def _sqrt32_exact(q: Fraction) -> float:
    y = struct.unpack("<f", struct.pack("<f", math.sqrt(float(q))))[0]
    # walk to the binary32 value whose rounding interval holds sqrt(q)
    for _ in range(4):
        lo = struct.unpack("<f", struct.pack("<I", struct.unpack("<I", struct.pack("<f", y))[0] - 1))[0]
        hi = struct.unpack("<f", struct.pack("<I", struct.unpack("<I", struct.pack("<f", y))[0] + 1))[0]
        mlo = (Fraction(lo) + Fraction(y)) / 2
        mhi = (Fraction(y) + Fraction(hi)) / 2
        if mlo * mlo > q:
            y = lo
        elif mhi * mhi < q:
            y = hi
        else:
            # ties (sqrt(q) exactly on a midpoint) cannot occur for a rational
            # square root of a ratio of binary32 values with a 24-bit result
            return y
    raise AssertionError("sqrt rounding did not settle")


def w8a8_forward(X, qw_kn, sw, bias):
    """W8A8 linear element by element; returns (qx, sx, acc, y_bf16)."""
    M, K = len(X), len(X[0])
    N = len(qw_kn[0])
    flat = [X[m][k] for m in range(M) for k in range(K)]
    codes, sx = quantize_group(flat, 127)
    qx = [codes[m * K:(m + 1) * K] for m in range(M)]
    acc = [[sum(qx[m][k] * qw_kn[k][n] for k in range(K)) for n in range(N)] for m in range(M)]
    y = [[bf16_exact(Fraction(acc[m][n]) * Fraction(sx) * Fraction(sw) +
                     (Fraction(bias[n]) if bias is not None else 0))
          for n in range(N)] for m in range(M)]
    return qx, sx, acc, y


def w4a16_forward(X, W, bias, group=64):
    """W4A16 linear element by element from the unquantized weight: each
    column's K-groups quantized with ``quantize_group`` (grid [-7, 7]), then
    y[m][n] = bf16(sum_k x[m][k] code[k][n] scale[k // G][n] + bias[n]) summed
    exactly. Returns (qw [K][N], sw [G][N], y [M][N])."""
    M, K = len(X), len(X[0])
    N = len(W[0])
    G = K // group
    qw = [[0] * N for _ in range(K)]
    sw = [[0.0] * N for _ in range(G)]
    for n in range(N):
        for g in range(G):
            codes, scale = quantize_group([W[k][n] for k in range(g * group, (g + 1) * group)], 7)
            for i, c in enumerate(codes):
                qw[g * group + i][n] = c
            sw[g][n] = scale
    y = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(X[m][k]) * Fraction(qw[k][n]) * Fraction(sw[k // group][n])
            if bias is not None:
                acc += Fraction(bias[n])
            row.append(bf16_exact(acc))
        y.append(row)
    return qw, sw, y


# ---- MXFP4 (OCP microscaling, FP4 E2M1 elements, E8M0 block scales) ----

_E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
         Fraction(4), Fraction(6)]


def e2m1_code(v: Fraction) -> int:
    """Nearest E2M1 value of an exact rational, ties to the even mantissa
    (codes 0, 2, 4, 6 have mantissa 0), magnitudes beyond 6 -> 6, zero -> +0."""
    m = abs(Fraction(v))
    best = None
    for c, g in enumerate(_E2M1):
        d = abs(m - g)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    if c == 0:
        return 0
    return c + (8 if v < 0 else 0)


def e2m1_value(code: int) -> Fraction:
    return -_E2M1[code & 7] if code & 8 else _E2M1[code & 7]


def mx_block(values):
    """One MX block: e with 2^(e+2) <= amax < 2^(e+3) (found by exact
    comparison), clamped to [-127, 127], -127 for an all-zero block; codes of
    v / 2^e. Returns (codes, e)."""
    amax = max(abs(Fraction(v)) for v in values)
    if amax == 0:
        return [0] * len(values), -127
    e = 0
    while Fraction(2) ** (e + 2) > amax:
        e -= 1
    while Fraction(2) ** (e + 3) <= amax:
        e += 1
    e = max(-127, min(127, e))
    return [e2m1_code(Fraction(v) / Fraction(2) ** e) for v in values], e


def mx_forward(Xh, R, T, L2, bias, block=32, out="bf16"):
    """MXFP4 main product plus low-rank and bias, element by element.
    Xh [M][K] smoothed activations (fp32 values), R [K][N] residual (fp32
    values), T [M][r], L2 [r][N]. Returns (qx, ex, qw [N][K], ew [N][K/B], y)."""
    M, K = len(Xh), len(Xh[0])
    N = len(R[0])
    r = len(L2)
    qx, ex = [], []
    for m in range(M):
        codes, es = [], []
        for b in range(K // block):
            c, e = mx_block(Xh[m][b * block:(b + 1) * block])
            codes += c
            es.append(e)
        qx.append(codes)
        ex.append(es)
    qw, ew = [], []
    for n in range(N):
        codes, es = [], []
        for b in range(K // block):
            c, e = mx_block([R[k][n] for k in range(b * block, (b + 1) * block)])
            codes += c
            es.append(e)
        qw.append(codes)
        ew.append(es)
    y = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                b = k // block
                acc += (e2m1_value(qx[m][k]) * Fraction(2) ** ex[m][b]) * \
                       (e2m1_value(qw[n][k]) * Fraction(2) ** ew[n][b])
            for j in range(r):
                acc += Fraction(T[m][j]) * Fraction(L2[j][n])
            if bias is not None:
                acc += Fraction(bias[n])
            row.append(rn32_exact(acc) if out == "f32" else bf16_exact(acc))
        y.append(row)
    return qx, ex, qw, ew, y
