"""Pins of the MLP-pair oracle's GELU (oracle/mlp.py): against an independent
evaluation of erf to 200 significant digits (Python's decimal module: the
power series of erf, pi by Machin's formula) with exact rational rounding to
bf16, closed-form bounds for the tails, and planted mistakes that must fail."""

import decimal
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute, mlp
from oracle import svdquant as sq

PREC = 200


def _pi():
    """pi = 16 atan(1/5) - 4 atan(1/239) (Machin), in the current context."""
    def atan_inv(x):
        x = Decimal(x)
        total, k, term = Decimal(0), 0, 1 / x
        eps = Decimal(10) ** -(PREC + 5)
        while abs(term) > eps:
            total += term / (2 * k + 1)
            k += 1
            term = -term / (x * x)
        return total
    return 16 * atan_inv(5) - 4 * atan_inv(239)


def gelu_decimal(y: float) -> Decimal:
    """GELU(y) = (y / 2)(1 + erf(y / sqrt 2)) with erf(z) = 2 / sqrt(pi)
    sum_n (-1)^n z^(2n+1) / (n! (2n+1)), to about 200 digits (enough for the
    cancellation in 1 + erf at y >= -16, whose terms reach 1e56)."""
    with decimal.localcontext() as ctx:
        ctx.prec = PREC
        z = Decimal(y) / Decimal(2).sqrt()
        z2 = z * z
        term, n, s = z, 0, Decimal(0)  # term = (-1)^n z^(2n+1) / n!
        eps = Decimal(10) ** -(PREC + 5)
        while True:
            s += term / (2 * n + 1)
            n += 1
            term = -term * z2 / n
            if abs(term) < eps and n > z2:
                break
        erf = 2 / _pi().sqrt() * s
        return Decimal(y) / 2 * (1 + erf)


def exact_bf16(y: float) -> float:
    v = Fraction(gelu_decimal(y))
    lo = brute.bf16_exact(v * (1 - Fraction(1, 10 ** 60)))
    hi = brute.bf16_exact(v * (1 + Fraction(1, 10 ** 60)))
    assert lo == hi, y  # 60 digits decide every rounding here
    return brute.bf16_exact(v)


def bf16_values(exp_lo, exp_hi, step=1):
    """bf16 values of both signs with exponent field in [exp_lo, exp_hi]."""
    out = []
    for s in (0, 1):
        for e in range(exp_lo, exp_hi + 1):
            for m in range(0, 128, step):
                out.append((s << 15) | (e << 7) | m)
    return sq.bf16_from_bits(np.array(out, dtype=np.uint16))


MID = bf16_values(118, 130)  # every bf16 value with 2^-9 <= |y| < 16


def test_gelu_matches_200_digit_evaluation_mid_range():
    got = mlp.gelu_bf16(MID)
    want = np.array([exact_bf16(float(y)) for y in MID])
    assert np.array_equal(got, want)


def test_gelu_small_arguments_round_to_half():
    # |y| < 2^-9: GELU(y) = (y / 2)(1 + d), |d| < 0.8 |y|, within half a bf16
    # ulp of y / 2; the 200-digit evaluation agrees on a sample
    ys = bf16_values(2, 117, step=17)
    assert np.array_equal(mlp.gelu_bf16(ys), ys / 2)
    for y in ys[::40]:
        assert exact_bf16(float(y)) == float(y) / 2


def test_gelu_tiny_ties_round_up():
    # y = k 2^-133 with k odd: y / 2 is a tie of the subnormal grid, and
    # GELU(y) > y / 2 decides it upward
    k = np.array([1, 3, 5, 127, 129, 255])
    for sgn in (1.0, -1.0):
        y = sgn * k * 2.0 ** -133
        want = np.ceil(sgn * k / 2.0) * 2.0 ** -133  # toward +inf from the tie
        assert np.array_equal(mlp.gelu_bf16(y), want)
    assert exact_bf16(3 * 2.0 ** -133) == 2 * 2.0 ** -133
    assert exact_bf16(-3 * 2.0 ** -133) == -1 * 2.0 ** -133


def test_gelu_tails_and_specials():
    big = bf16_values(131, 140, step=9)
    g = mlp.gelu_bf16(big)
    pos = big > 0
    # y Phi(-y) < e^-128 relative for y >= 16: rounds to y; for y <= -16
    # |GELU| < 16 e^-128 < 2^-134: rounds to -0
    assert np.array_equal(g[pos], big[pos])
    assert np.all(g[~pos] == 0) and np.all(np.signbit(g[~pos]))
    with np.errstate(invalid="ignore"):
        sp = mlp.gelu_bf16(np.array([0.0, -0.0, np.inf, -np.inf, np.nan]))
    assert sp[0] == 0 and not np.signbit(sp[0]) and sp[1] == 0 and np.signbit(sp[1])
    assert sp[2] == np.inf and np.isnan(sp[3]) and np.isnan(sp[4])
    # the boundaries of the mid range against the decimal evaluation
    for y in (2.0 ** -9, -(2.0 ** -9), 15.9375, -15.9375, -13.25, -13.0):
        assert mlp.gelu_bf16(np.array([y]))[0] == exact_bf16(y), y


def _tanh_form(y):
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (y + 0.044715 * y ** 3)))


def _one_plus_erf(y):
    from scipy.special import erf
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + erf(y / np.sqrt(2.0)))


@pytest.mark.parametrize("mutant", [_tanh_form, _one_plus_erf])
def test_planted_gelu_mistakes_fail(monkeypatch, mutant):
    monkeypatch.setattr(mlp, "gelu_exact64", mutant)
    with pytest.raises((AssertionError, ArithmeticError)):
        test_gelu_matches_200_digit_evaluation_mid_range()


def test_down_activation_side_composes_the_pinned_steps():
    rng = np.random.default_rng(5)
    M, N, r = 6, 128, 16
    y = sq.bf16_round(rng.standard_normal((M, N)) * 2.0)
    s = sq.rn32(np.exp(rng.standard_normal(N) * 0.3))
    L1s = sq.bf16_round(rng.standard_normal((N, r)) * 0.1)
    side = mlp.down_activation_side(y, {"s": s, "L1s": L1s})
    g = mlp.gelu_bf16(y)
    assert np.array_equal(side["g"], g)
    qx, sx = sq.quantize_activations(g, s)
    assert np.array_equal(side["qx"], qx) and np.array_equal(side["sx"], sx)
    assert np.array_equal(side["T"], sq.lowrank_down(g, L1s))
