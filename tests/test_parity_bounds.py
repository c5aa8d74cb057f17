"""The per-element bounds the GPU parity tests apply (tests/parity_bounds.py),
checked on the CPU against an fp32 emulation of the device's order of
operations: the emulation stays inside them, and plausible device mistakes
(a dropped group, a scale taken from the wrong row, a dropped bias, a
dropped low-rank term, a misplaced output tile) fall outside."""

import numpy as np
import pytest

from bit_quantized_linear_amd import workloads as wl
from oracle import svdquant as sq
from oracle import w8a8 as o8
from tests import parity_bounds as PB

F64 = np.float64


def rn32(x):
    return np.asarray(x, dtype=F64).astype(np.float32).astype(F64)


def emulate_w4a4(qx, sx, qw, sw, T, L2, bias, out, drop_group=None, sx_row_shift=0, drop_bias=False,
                 drop_lowrank=False):
    """fp32 evaluation in the device's order: per group acc = fl(fl(sx sw) P +
    acc), then the low-rank products one by one, then the bias, then one
    rounding to the output type."""
    M, K = qx.shape
    N = qw.shape[1]
    acc = np.zeros((M, N))
    for g in range(K // 64):
        if g == drop_group:
            continue
        sl = slice(64 * g, 64 * g + 64)
        P = qx[:, sl].astype(F64) @ qw[sl].astype(F64)
        sxg = np.roll(sx[g], sx_row_shift)
        C = rn32(sxg[:, None].astype(F64) * sw[g][None, :].astype(F64))
        acc = rn32(C * P + acc)
    if T is not None and not drop_lowrank:
        for j in range(T.shape[1]):
            acc = rn32(acc + T[:, j:j + 1] * L2[j:j + 1, :])
    if bias is not None and not drop_bias:
        acc = rn32(acc + bias[None, :])
    return sq.round_output(acc, out)


@pytest.fixture(scope="module")
def problem():
    rng = np.random.default_rng(3)
    M, K, N, r = 48, 320, 40, 16
    X = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32)))
    X[:, 7] *= 20
    X = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(X)).astype(F64)
    W = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32((0.02 * rng.standard_normal((K, N))).astype(np.float32)))
    bias = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32((0.01 * rng.standard_normal(N)).astype(np.float32)))
    prep = sq.prepare_weights(W.astype(F64), sq.channel_absmax(X), r)
    return X, prep, bias.astype(F64)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fp32_device_order_stays_inside_the_bound(problem, out):
    X, prep, bias = problem
    ref = sq.forward(X, prep, bias, out)
    got = emulate_w4a4(ref["qx"], ref["sx"], prep["qw"], prep["sw"], ref["T"], prep["L2"], bias, out)
    tol = PB.w4a4_tolerance(ref["qx"], ref["sx"], prep["qw"], prep["sw"], ref["T"], prep["L2"], bias, got,
                            ref["y"], out)
    PB.check_elementwise(got, ref["y"], tol)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("mistake", ["drop_group", "sx_row_shift", "drop_bias", "drop_lowrank", "tile_swap"])
def test_device_mistakes_fall_outside_the_bound(problem, out, mistake):
    X, prep, bias = problem
    ref = sq.forward(X, prep, bias, out)
    kw = {"drop_group": {"drop_group": 2}, "sx_row_shift": {"sx_row_shift": 1}, "drop_bias": {"drop_bias": True},
          "drop_lowrank": {"drop_lowrank": True}, "tile_swap": {}}[mistake]
    got = emulate_w4a4(ref["qx"], ref["sx"], prep["qw"], prep["sw"], ref["T"], prep["L2"], bias, out, **kw)
    if mistake == "tile_swap":
        got = got.copy()
        got[[3, 4]] = got[[4, 3]]  # two output rows stored in each other's place
    tol = PB.w4a4_tolerance(ref["qx"], ref["sx"], prep["qw"], prep["sw"], ref["T"], prep["L2"], bias, got,
                            ref["y"], out)
    with pytest.raises(AssertionError, match="outside the bound"):
        PB.check_elementwise(got, ref["y"], tol)


def test_w8a8_bound():
    rng = np.random.default_rng(9)
    X = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32(rng.standard_normal((40, 192)).astype(np.float32)))
    W = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32((0.02 * rng.standard_normal((192, 24))).astype(np.float32)))
    bias = wl.f32_from_bf16_bits(wl.bf16_bits_from_f32((0.01 * rng.standard_normal(24)).astype(np.float32)))
    qw, sw = o8.prepare_weights(W)
    ref = o8.forward(X, qw, sw, bias)
    s32 = rn32(float(ref["sx"]) * float(sw))
    dev = sq.bf16_round(rn32(rn32(rn32(ref["acc"].astype(F64)) * s32) + bias[None, :]))
    tol = PB.w8a8_tolerance(ref["acc"], ref["sx"], sw, bias, dev, ref["y"])
    PB.check_elementwise(dev, ref["y"], tol)
    bad = sq.bf16_round(rn32(rn32(rn32(ref["acc"].astype(F64)) * s32)))  # bias dropped
    tol = PB.w8a8_tolerance(ref["acc"], ref["sx"], sw, bias, bad, ref["y"])
    with pytest.raises(AssertionError, match="outside the bound"):
        PB.check_elementwise(bad, ref["y"], tol)


def test_subnormal_scale_products_stay_inside_the_bound(problem):
    """Rows scaled far down (2^-120): fl(sx sw) falls into fp32's subnormal
    range, where its rounding error is absolute; the fp32 emulation must
    still be inside the bound."""
    X, prep, bias = problem
    Xs = X.copy()
    Xs[2] *= 2.0 ** -120
    Xs[5] *= 2.0 ** -110
    ref = sq.forward(Xs, prep, None, "f32")
    prod = ref["sx"][:, 2][:, None].astype(F64) * prep["sw"].astype(F64)
    assert np.any((prod > 0) & (prod < 2.0 ** -126))
    got = emulate_w4a4(ref["qx"], ref["sx"], prep["qw"], prep["sw"], ref["T"], prep["L2"], None, "f32")
    tol = PB.w4a4_tolerance(ref["qx"], ref["sx"], prep["qw"], prep["sw"], ref["T"], prep["L2"], None, got,
                            ref["y"], "f32")
    PB.check_elementwise(got, ref["y"], tol)


def test_scale_folded_with_the_unpack_factor_falls_outside_for_tiny_rows(problem):
    """A device that folds the 1/256 of the 16 * code nibble unpack into the
    activation scale (fl(fl(sx / 256) sw) times 256 P) pushes the scale
    products of tiny rows 8 binades deeper into fp32's subnormal range; the
    bound flags it, while the product rounded where the formula rounds it
    passes (test above)."""
    X, prep, bias = problem
    Xs = X.copy()
    Xs[2] *= 2.0 ** -120
    ref = sq.forward(Xs, prep, None, "f32")
    M, K = ref["qx"].shape
    acc = np.zeros((M, prep["qw"].shape[1]))
    for g in range(K // 64):
        sl = slice(64 * g, 64 * g + 64)
        P = ref["qx"][:, sl].astype(F64) @ prep["qw"][sl].astype(F64)
        C = rn32(rn32(ref["sx"][g].astype(F64) / 256)[:, None] * prep["sw"][g][None, :].astype(F64))
        acc = rn32(C * (256 * P) + acc)
    for j in range(ref["T"].shape[1]):
        acc = rn32(acc + ref["T"][:, j:j + 1] * prep["L2"][j:j + 1, :])
    got = sq.round_output(acc, "f32")
    tol = PB.w4a4_tolerance(ref["qx"], ref["sx"], prep["qw"], prep["sw"], ref["T"], prep["L2"], None, got,
                            ref["y"], "f32")
    with pytest.raises(AssertionError, match="outside the bound"):
        PB.check_elementwise(got, ref["y"], tol)
