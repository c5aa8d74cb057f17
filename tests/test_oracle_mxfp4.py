"""Pins of the MXFP4 oracle (CPU only): a hand-derived rounding table, exact
rational brute force of the whole linear, power-of-two invariance, on-grid
exactness, idempotence, and planted mistakes that must fail a pin."""

from fractions import Fraction

import numpy as np
import pytest

from bit_quantized_linear_amd import workloads as wl
from oracle import brute
from oracle import mxfp4 as mx
from oracle import svdquant as sq
from tests.oracle_pins import load_golden

F64 = np.float64


def _bf16(a):
    return wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(np.asarray(a, np.float32))).astype(F64)


def test_golden_e2m1_rounding_and_exponents():
    g = load_golden("mxfp4_rounding.txt")
    r = mx.e2m1_round(g["q"])
    assert list(r) == g["r"]
    assert [int(c) for c in mx.e2m1_encode(r)] == [int(c) for c in g["code"]]
    assert [int(e) for e in mx.shared_exponent(g["amax"])] == [int(e) for e in g["e"]]


def test_e2m1_rounding_matches_exact_brute_force_on_a_dense_grid():
    # every multiple of 1/64 in [-8, 8] (all ties and midpoints included)
    q = np.arange(-512, 513) / 64.0
    got = mx.e2m1_encode(mx.e2m1_round(q))
    ref = [brute.e2m1_code(Fraction(int(v * 64), 64)) for v in q]
    assert [int(c) for c in got] == ref
    assert np.array_equal(mx.e2m1_decode(got), [float(brute.e2m1_value(c)) for c in ref])


def test_block_exponents_match_brute_force():
    rng = np.random.default_rng(3)
    vals = np.concatenate([np.ldexp(rng.uniform(1, 2, 40), rng.integers(-140, 120, 40)),
                           [2.0 ** -149, 6.0, 7.999999, 8.0, 0.0]]).astype(np.float32).astype(F64)
    for v in vals:
        _, e = brute.mx_block([v])
        assert int(mx.shared_exponent(v)) == e, v


def test_brute_force_mxfp4_linear():
    rng = np.random.default_rng(31)
    M, K, N, r = 3, 64, 4, 2
    X = _bf16(rng.standard_normal((M, K)))
    X[:, 5] *= 20
    W = _bf16(0.02 * rng.standard_normal((K, N)))
    W[32:, 3] = 0.0  # an all-zero block
    s = sq.smoothing_factors(sq.channel_absmax(X), W)
    L1s = sq.bf16_round(rng.standard_normal((K, r)) * 0.01)
    L1s[32:, :] = 0.0  # with W[32:, 3] = 0 the residual block (k >= 32, n = 3) is zero
    L2 = sq.bf16_round(rng.standard_normal((r, N)) * 0.01)
    b = _bf16(0.01 * rng.standard_normal(N))
    prep = mx.prepare_from_factors(W, s, L1s, L2)
    out = mx.forward(X, prep, b, "f32")
    Xh = sq.smooth_activations(X, s).astype(F64)
    qx_b, ex_b, qw_b, ew_b, y_b = brute.mx_forward(Xh.tolist(), np.asarray(prep["R32"], F64).tolist(),
                                                   np.asarray(out["T"]).tolist(), L2.tolist(), b.tolist(),
                                                   out="f32")
    assert np.array_equal(out["qx"], np.array(qx_b)) and np.array_equal(out["ex"], np.array(ex_b))
    assert np.array_equal(prep["qw"], np.array(qw_b)) and np.array_equal(prep["ew"], np.array(ew_b))
    assert prep["ew"][3, 1] == -127 and not prep["qw"][3, 32:].any()
    assert np.array_equal(out["y"], np.array(y_b))


def test_power_of_two_scaling_moves_only_the_exponents():
    rng = np.random.default_rng(4)
    V = rng.standard_normal((5, 96)).astype(np.float32).astype(F64)
    c1, e1 = mx.quantize_rows(V)
    c2, e2 = mx.quantize_rows(V * 2.0 ** 7)
    c3, e3 = mx.quantize_rows(-V)
    assert np.array_equal(c1, c2) and np.array_equal(e2, e1 + 7)
    nz = mx.e2m1_decode(c1) != 0
    assert np.array_equal(mx.e2m1_decode(c3)[nz], -mx.e2m1_decode(c1)[nz]) and np.array_equal(e3, e1)


def test_on_grid_values_are_exact_and_requantization_is_idempotent():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, (4, 64)).astype(np.uint8)
    codes[:, ::32] = 7  # a 6 in every block: the block exponent is the chosen one
    e = rng.integers(-20, 20, (4, 2))
    V = mx.dequantize_rows(codes, e)
    c2, e2 = mx.quantize_rows(V)
    assert np.array_equal(e2, e)
    assert np.array_equal(mx.e2m1_decode(c2), mx.e2m1_decode(codes))  # -0 comes back as +0
    c3, e3 = mx.quantize_rows(mx.dequantize_rows(c2, e2))
    assert np.array_equal(c3, c2) and np.array_equal(e3, e2)


def test_main_product_is_dequantize_then_matmul():
    case = wl.CASES["tiny"]
    X = wl.activations(case)["values"].astype(F64)
    W = wl.weight(case)["values"].astype(F64)
    prep = mx.prepare_weights(W, sq.channel_absmax(X), 16)
    out = mx.forward(X, prep, None)
    A = mx.dequantize_rows(out["qx"], out["ex"])
    B = mx.dequantize_rows(prep["qw"], prep["ew"])
    ref = A @ B.T + np.asarray(out["T"], F64) @ prep["L2"]
    assert np.max(np.abs(out["y64"] - ref)) <= 1e-12 * np.max(np.abs(ref))
    # the method's accuracy against X W, reported only (parity unpinned)
    rel = np.linalg.norm(out["y64"] - X @ W) / np.linalg.norm(X @ W)
    assert rel < 0.5


# ---- planted mistakes --------------------------------------------------------

def _mut_ties_away(q):
    q = np.asarray(q, dtype=F64)
    m = np.abs(q)
    rnd = lambda t: np.floor(t + 0.5)  # noqa: E731
    r = np.where(m < 2.0, rnd(2.0 * m) / 2.0, np.where(m < 4.0, rnd(m), 2.0 * rnd(m / 2.0)))
    r = np.minimum(r, 6.0)
    return np.where(q < 0, -r, r)


def _mut_emax_3(amax):
    amax = np.asarray(amax, dtype=F64)
    _, x = np.frexp(amax)
    return np.clip(np.where(amax > 0, x - 1 - 3, -127), -127, 127).astype(np.int64)


def _mut_ceil_log2(amax):
    amax = np.asarray(amax, dtype=F64)
    e = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    return np.clip(e, -127, 127).astype(np.int64)


@pytest.mark.parametrize("name,mutant", [
    ("e2m1_round", _mut_ties_away),
    ("shared_exponent", _mut_emax_3),
    ("shared_exponent", _mut_ceil_log2),
])
def test_planted_mistakes_fail_a_pin(monkeypatch, name, mutant):
    monkeypatch.setattr(mx, name, mutant)
    failed = 0
    for pin in (test_golden_e2m1_rounding_and_exponents,
                test_e2m1_rounding_matches_exact_brute_force_on_a_dense_grid,
                test_block_exponents_match_brute_force, test_brute_force_mxfp4_linear):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
