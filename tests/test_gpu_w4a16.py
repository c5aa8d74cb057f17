"""W4A16 linear (the awq_w4a16 layer type): HIP path vs the CPU oracle,
through the C-ABI (needs an MI355X).

Weights are prepared by the library on the host (its container is checked
byte for byte against the oracle's codes and scales by the CPU tests) and
the device output is compared with oracle.w4a16.forward on the oracle's own
codes: rel-L2 <= 1e-3, cosine >= 0.99999, all finite, and every element
within one bf16 ulp plus an a-priori bound of the kernel's fp32 evaluation.
"""

import sys

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b
from bit_quantized_linear_amd import workloads as wl
from oracle import svdquant as sq
from oracle import w4a16 as o16
from tests import gpu_harness as H
from tests.oracle_pins import cosine, rel_l2

pytestmark = pytest.mark.gpu

F64 = np.float64


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert b.svdq_check_device(torch.cuda.current_device()) == b.SVDQ_OK, "not a gfx950 device"


def run(Xbits, packed, bias_bits, N):
    t = H.torch()
    M = Xbits.shape[0]
    Y = t.full((M, N), -1, dtype=t.int16, device="cuda")  # NaN pattern 0xFFFF: unwritten is visible
    b.w4a16_linear(H.dev(Xbits), H.dev(packed), H.dev(bias_bits) if bias_bits is not None else None, Y, N)
    t.cuda.synchronize()
    return Y


def check(Y, X, qw, sw, bias):
    """rel-L2 / cosine bar plus a per-element bound: one bf16 ulp of the
    oracle's value, plus the error of the kernel's fp32 evaluation. Per group
    the MFMA sums x (136 + q) onto -136 S (S = sum x), so its rounding is at
    most ~(64 + 16) fp32 ulps of 136 sum |x|; the groups are then added in
    fp32 (G + 4 ulps of sum |x q sw|)."""
    y = sq.bf16_from_bits(H.host(Y).view(np.uint16))
    ref = o16.forward(X, qw, sw, bias)
    assert np.all(np.isfinite(y))
    K = X.shape[1]
    G = K // 64
    absx = np.abs(np.asarray(X, dtype=F64))
    s_rep = np.repeat(np.abs(np.asarray(sw, dtype=F64)), 64, axis=0)
    a1 = absx @ s_rep
    a2 = absx @ np.abs(o16.dequantize(qw, sw))
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref["y"]), 1e-30))[1] - 8)
    tol = ulp + 2.0 ** -24 * (136 * 80 * a1 + (G + 4) * a2)
    bad = np.abs(y - ref["y"]) > tol
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5].tolist(), y[bad][:5], ref["y"][bad][:5])
    r, c = rel_l2(y, ref["y"]), cosine(y, ref["y"])
    assert r <= 1e-3 and c >= 0.99999, (r, c)
    return y, ref, float(np.mean(y != ref["y"]))


def problem(M, K, N, seed, bias=True, outliers=0):
    X = wl.random_bf16(seed * 10 + 1, (M, K))
    Xv = X["values"].copy()
    if outliers:
        rng = np.random.default_rng(seed)
        Xv[:, rng.choice(K, outliers, replace=False)] *= 20.0
    Xb = wl.bf16_bits_from_f32(Xv)
    W = wl.random_bf16(seed * 10 + 2, (K, N), 0.02)
    Wv = W["values"].copy()
    Wv[:, ::7] *= 8.0  # heavy columns
    Wb = wl.bf16_bits_from_f32(Wv)
    bb = wl.random_bf16(seed * 10 + 3, (N,), 0.01)["bits"] if bias else None
    return Xb, Wb, bb


@pytest.mark.parametrize("M,K,N", [
    (1, 64, 16), (2, 64, 1), (2, 192, 40), (3, 320, 100), (5, 128, 33),
    (16, 1024, 96), (17, 512, 64), (33, 256, 72), (2, 3072, 544), (1, 4096, 1000),
    # rows of X per block limited by LDS: 2 (K = 12288, 3 chunks), 1 (K = 28672);
    # few column pairs at large K; an odd group count at large K
    (5, 12288, 64), (3, 14336, 40), (2, 28672, 48), (2, 12288, 3072), (2, 12224, 80),
    # more than 8 rows per block: two tiles per block (and 8 waves with few blocks)
    (40, 3072, 1024), (12, 4096, 256),
])
def test_w4a16_matches_oracle(M, K, N):
    say(f"w4a16 M={M} K={K} N={N}")
    Xb, Wb, bb = problem(M, K, N, seed=M * 31 + K + N, outliers=max(1, K // 200))
    packed = b.w4a16_prepare_weights(Wb)
    Wf = wl.f32_from_bf16_bits(Wb)
    qw, sw = o16.prepare_weights(Wf)
    Y = run(Xb, packed, bb, N)
    y, ref, mism = check(Y, wl.f32_from_bf16_bits(Xb), qw, sw,
                         None if bb is None else wl.f32_from_bf16_bits(bb))
    say(f"  rel-L2 {rel_l2(y, ref['y']):.2e}, bf16 mismatches {mism:.4%}")


def test_w4a16_no_bias_and_zero_rows():
    Xb, Wb, _ = problem(6, 256, 48, seed=3, bias=False)
    Xv = wl.f32_from_bf16_bits(Xb).copy()
    Xv[2] = 0.0
    Xb = wl.bf16_bits_from_f32(Xv)
    packed = b.w4a16_prepare_weights(Wb)
    qw, sw = o16.prepare_weights(wl.f32_from_bf16_bits(Wb))
    Y = run(Xb, packed, None, 48)
    y, _, _ = check(Y, wl.f32_from_bf16_bits(Xb), qw, sw, None)
    assert not y[2].any()


def test_w4a16_modulation_full_size_all_outputs():
    """The modulation workload at its full size (M = 2, K = 3072, N = 18432),
    every output against the oracle, twice (deterministic)."""
    case = wl.CASES["modulation"]
    say(f"w4a16 modulation M={case.M} K={case.K} N={case.N}")
    X = wl.activations(case)
    W = wl.weight(case)
    bias = wl.bias(case)
    packed = b.w4a16_prepare_weights(W["bits"])
    qw, sw = o16.prepare_weights(W["values"])
    Y = run(X["bits"], packed, bias["bits"], case.N)
    y, ref, mism = check(Y, X["values"], qw, sw, bias["values"])
    say(f"  rel-L2 {rel_l2(y, ref['y']):.2e}, bf16 mismatches {mism:.4%}")
    Y2 = run(X["bits"], packed, bias["bits"], case.N)
    assert np.array_equal(H.host(Y), H.host(Y2))


def test_w4a16_larger_batch_sampled_rows():
    """M = 300 (19 batch chunks, ragged last) at K = 3072, N = 1024: sampled
    rows against the oracle."""
    M, K, N = 300, 3072, 1024
    Xb, Wb, bb = problem(M, K, N, seed=9, outliers=15)
    packed = b.w4a16_prepare_weights(Wb)
    qw, sw = o16.prepare_weights(wl.f32_from_bf16_bits(Wb))
    Y = run(Xb, packed, bb, N)
    rows = np.array([0, 15, 16, 17, 150, 287, 288, 299])
    Xv = wl.f32_from_bf16_bits(Xb)
    yall = H.host(Y)
    t = H.torch()
    sub = t.from_numpy(np.ascontiguousarray(yall[rows]))
    check(sub, Xv[rows], qw, sw, wl.f32_from_bf16_bits(bb))


def test_w4a16_empty_batch_launches_nothing():
    t = H.torch()
    Wb = wl.random_bf16(5, (128, 16), 0.02)["bits"]
    packed = H.dev(b.w4a16_prepare_weights(Wb))
    X = t.empty((0, 128), dtype=t.int16, device="cuda")
    Y = t.empty((0, 16), dtype=t.int16, device="cuda")
    b.w4a16_linear(X, packed, None, Y, 16)
    t.cuda.synchronize()
