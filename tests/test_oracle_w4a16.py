"""Pins of the W4A16 oracle (CPU only): brute force in exact rational
arithmetic, a hand-derived golden file, on-grid weights against a plain
matmul, invariants, and planted mistakes that must fail a pin."""

import numpy as np
import pytest

from bit_quantized_linear_amd import workloads as wl
from oracle import brute
from oracle import svdquant as sq
from oracle import w4a16 as o16
from tests.oracle_pins import load_golden

F64 = np.float64


def _bf16(a):
    return wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(np.asarray(a, np.float32))).astype(F64)


def _triples(vals, shape):
    out = np.zeros(shape)
    t = np.array(vals).reshape(-1, 3)
    for r, c, v in t:
        out[int(r), int(c)] = v
    return out


def _golden():
    g = load_golden("w4a16_tiny.txt")
    W = _triples(g["w_nz"], (64, 2))
    X = _triples(g["x_nz"], (2, 64))
    return g, X, W


def test_golden_w4a16_tiny():
    g, X, W = _golden()
    qw, sw = o16.prepare_weights(W)
    assert list(sw.ravel()) == g["sw"]
    assert np.array_equal(qw, _triples(g["qw_nz"], (64, 2)))
    out = o16.forward(X, qw, sw, np.array(g["bias"]))
    assert list(out["y"].ravel()) == g["y"]


def test_brute_force_w4a16():
    rng = np.random.default_rng(41)
    M, K, N = 3, 128, 5
    X = _bf16(rng.standard_normal((M, K)))
    X[:, 9] *= 20
    W = _bf16(0.02 * rng.standard_normal((K, N)))
    W[:, 2] *= 8
    W[64:, 4] = 0.0  # an all-zero group
    b = _bf16(0.01 * rng.standard_normal(N))
    qw, sw = o16.prepare_weights(W)
    qw_b, sw_b, y_b = brute.w4a16_forward(X.tolist(), W.tolist(), b.tolist())
    assert np.array_equal(qw, np.array(qw_b))
    assert np.array_equal(sw.astype(F64), np.array(sw_b))
    assert sw[1, 4] == 0 and not qw[64:, 4].any()
    out = o16.forward(X, qw, sw, b)
    assert np.array_equal(out["y"], np.array(y_b))


def test_on_grid_weights_are_kept_and_match_a_plain_matmul():
    """Weights already on the INT4 grid (code times a power-of-two scale,
    with a +-7 in every group) quantize to themselves, and the linear equals
    bf16(X W + bias) computed by one matmul of the raw weight."""
    rng = np.random.default_rng(5)
    M, K, N = 4, 192, 7
    codes = rng.integers(-7, 8, (K, N))
    codes[::64, :] = 7
    scale = 2.0 ** rng.integers(-9, -4, (K // 64, N))
    W = codes * np.repeat(scale, 64, axis=0)
    qw, sw = o16.prepare_weights(W)
    assert np.array_equal(qw, codes) and np.array_equal(sw.astype(F64), scale)
    X = _bf16(rng.standard_normal((M, K)))
    b = _bf16(0.01 * rng.standard_normal(N))
    out = o16.forward(X, qw, sw, b)
    assert np.array_equal(out["y"], sq.bf16_round(X @ W + b[None, :]))


def test_requantizing_the_dequantized_weight_is_idempotent():
    rng = np.random.default_rng(6)
    W = _bf16(0.02 * rng.standard_normal((256, 9)))
    qw, sw = o16.prepare_weights(W)
    qw2, sw2 = o16.prepare_weights(o16.dequantize(qw, sw))
    assert np.array_equal(qw, qw2) and np.array_equal(sw, sw2)


def test_linearity_in_x_and_sign():
    rng = np.random.default_rng(7)
    X = _bf16(rng.standard_normal((5, 128)))
    W = _bf16(0.02 * rng.standard_normal((128, 6)))
    qw, sw = o16.prepare_weights(W)
    a = o16.forward(X, qw, sw)
    assert np.array_equal(o16.forward(4 * X, qw, sw)["y64"], 4 * a["y64"])
    assert np.array_equal(o16.forward(-X, qw, sw)["y64"], -a["y64"])
    qn, sn = o16.prepare_weights(-W)
    assert np.array_equal(qn, -qw) and np.array_equal(sn, sw)


# ---- planted mistakes: each must fail one of the pins above ----------------

def _mut_scale_interleaved(qw, sw, group=64):
    # scale of row k taken from group k % G instead of k // G
    qw = np.asarray(qw, dtype=F64)
    return qw * np.tile(np.asarray(sw, dtype=F64), (group, 1))


def _mut_dequant_drops_scale(qw, sw, group=64):
    return np.asarray(qw, dtype=F64)


def _mut_quantize_absmax_over_8(W, group=64):
    old = sq.QMAX
    try:
        sq.QMAX = 8
        return sq.quantize_weights(np.asarray(W, dtype=np.float32), group)
    finally:
        sq.QMAX = old


@pytest.mark.parametrize("name,mutant", [
    ("dequantize", _mut_scale_interleaved),
    ("dequantize", _mut_dequant_drops_scale),
    ("prepare_weights", _mut_quantize_absmax_over_8),
])
def test_planted_mistakes_fail_a_pin(monkeypatch, name, mutant):
    monkeypatch.setattr(o16, name, mutant)
    failed = 0
    for pin in (test_golden_w4a16_tiny, test_brute_force_w4a16,
                test_on_grid_weights_are_kept_and_match_a_plain_matmul):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
