"""Pins of the W8A8 oracle (CPU only)."""

import numpy as np

from bit_quantized_linear_amd import workloads as wl
from oracle import brute
from oracle import w8a8 as o8
from tests.oracle_pins import load_golden, rel_l2

F64 = np.float64


def test_golden_w8a8_tiny():
    g = load_golden("w8a8_tiny.txt")
    X = np.array(g["x"]).reshape(2, 3)
    W = np.array(g["w"]).reshape(3, 2)
    qw, sw = o8.prepare_weights(W)
    assert float(sw) == g["sw"][0]
    assert list(qw.ravel()) == g["qw"]
    out = o8.forward(X, qw, sw, np.array(g["bias"]))
    assert float(out["sx"]) == g["sx"][0]
    assert list(out["qx"].ravel()) == g["qx"]
    assert list(out["acc"].ravel()) == g["acc"]
    assert list(out["y"].ravel()) == g["y"]


def test_brute_force_w8a8():
    rng = np.random.default_rng(21)
    M, K, N = 8, 96, 12
    X = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))).astype(F64)
    X[:, 3] *= 10
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32).astype(F64)
    b = (0.01 * rng.standard_normal(N)).astype(np.float32).astype(F64)
    qw, sw = o8.prepare_weights(W)
    codes_b, sw_b = brute.quantize_group(W.ravel().tolist(), 127)
    assert float(sw) == sw_b and list(qw.ravel()) == codes_b
    out = o8.forward(X, qw, sw, b)
    qx_b, sx_b, acc_b, y_b = brute.w8a8_forward(X.tolist(), qw.tolist(), float(sw), b.tolist())
    assert float(out["sx"]) == sx_b
    assert np.array_equal(out["qx"], np.array(qx_b))
    assert np.array_equal(out["acc"], np.array(acc_b))
    assert np.array_equal(out["y"], np.array(y_b))


def test_w8a8_dequantize_then_matmul():
    case = wl.CASES["tiny"]
    X = wl.activations(case)["values"].astype(F64)
    W = wl.weight(case)["values"].astype(F64)
    qw, sw = o8.prepare_weights(W)
    out = o8.forward(X, qw, sw, None)
    ref = (out["qx"].astype(F64) * float(out["sx"])) @ (qw.astype(F64) * float(sw))
    assert rel_l2(out["y64"], ref) <= 1e-14
    assert np.abs(out["acc"]).max() < 2 ** 31


def test_w8a8_on_grid_exact_and_invariants():
    rng = np.random.default_rng(2)
    M, K, N = 10, 64, 6
    q = rng.integers(-127, 128, (M, K))
    q[3, 7] = -127
    X = q * 2.0 ** -3
    qx, sx = o8.quantize_activations(X)
    assert float(sx) == 2.0 ** -3 and np.array_equal(qx, q)
    W = (0.02 * rng.standard_normal((K, N))).astype(np.float32).astype(F64)
    qw, sw = o8.prepare_weights(W)
    a = o8.forward(X, qw, sw, None)
    b = o8.forward(X * 4, qw, sw, None)
    c = o8.forward(-X, qw, sw, None)
    assert np.array_equal(b["qx"], a["qx"]) and np.array_equal(b["y64"], a["y64"] * 4)
    assert np.array_equal(c["qx"], -a["qx"]) and np.array_equal(c["y64"], -a["y64"])


def test_w8a8_all_zero_tensor():
    X = np.zeros((3, 64))
    qx, sx = o8.quantize_activations(X)
    assert float(sx) == 0.0 and not qx.any()
