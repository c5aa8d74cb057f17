"""MXFP4 variant of the SVDQuant W4A4 linear: HIP path vs the CPU oracle,
through the C-ABI (needs an MI355X).

Codes and E8M0 scales of the activation pass bit-exact; T within one bf16
ulp plus the bound of an fp32 sum; outputs rel-L2 <= 1e-3, cosine >=
0.99999, all finite, and every element within one output ulp, one T step
times |L2|, and an a-priori bound of the kernel's fp32 accumulation. Inputs are prepared by the
oracle and written by the test-side container writer; nothing flows back.
"""

import sys

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b
from bit_quantized_linear_amd import workloads as wl
from oracle import mxfp4 as mx
from oracle import svdquant as sq
from tests import gpu_harness as H
from tests.mx_format import pack_mx_codes, pack_mx_scales, scale_ld, unpack_mx_codes, unpack_mx_scales
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


def problem(M, K, N, rank, seed, outliers=(), bias=True):
    X = wl.random_bf16(seed * 10 + 1, (M, K))
    Xv = X["values"].copy()
    for ch in outliers:
        Xv[:, ch] *= 20.0
    Xb = wl.bf16_bits_from_f32(Xv)
    Xv = wl.f32_from_bf16_bits(Xb).astype(F64)
    W = wl.random_bf16(seed * 10 + 2, (K, N), 0.02)
    Wv = W["values"].copy()
    Wv[:, ::11] *= 8.0
    bb = wl.random_bf16(seed * 10 + 3, (N,), 0.01) if bias else None
    prep = mx.prepare_weights(Wv.astype(F64), sq.channel_absmax(Xv), rank)
    return Xb, Xv, prep, bb


def run_act(Xb, prep, rank, split=True):
    t = H.torch()
    M, K = Xb.shape
    qx = t.empty((M, K // 2), dtype=t.uint8, device="cuda")
    ux = t.empty((K // 32, scale_ld(M)), dtype=t.uint8, device="cuda")
    T = t.empty((M, max(rank, 1)), dtype=t.int16, device="cuda") if rank else None
    l1t = H.dev(sq.bf16_bits(np.asarray(prep["L1s"]).T)) if rank else None
    b.svdq_mx_quantize_act(H.dev(Xb), H.dev(prep["s"].astype(np.float32)), l1t, qx, ux, T, rank,
                           workspace=H.act_workspace(M, K, rank) if split else None)
    t.cuda.synchronize()
    return qx, ux, T


def run_linear(qx, ux, T, prep, bias_bits, M, N, K, rank, out="bf16"):
    t = H.torch()
    Y = t.empty((M, N), dtype=t.float32 if out == "f32" else t.int16, device="cuda")
    qw = H.dev(pack_mx_codes(prep["qw"]))
    uw = H.dev(pack_mx_scales(prep["ew"]))
    l2t = H.dev(sq.bf16_bits(np.asarray(prep["L2"]).T)) if rank else None
    b.svdq_mx_linear(qx, ux, T, qw, uw, l2t, H.dev(bias_bits) if bias_bits is not None else None, Y, M, N, K,
                     rank)
    t.cuda.synchronize()
    return Y


def check_act(qx, ux, T, Xv, prep, rank):
    M, K = Xv.shape
    ref_q, ref_e = mx.quantize_activations(Xv, prep["s"])
    got_q = unpack_mx_codes(H.host(qx), K)
    got_e = unpack_mx_scales(H.host(ux), M)
    assert np.array_equal(got_e, ref_e), np.argwhere(got_e != ref_e)[:5]
    assert np.array_equal(got_q, ref_q), np.argwhere(got_q != ref_q)[:5]
    if rank:
        ref_T = sq.lowrank_down(Xv, prep["L1s"])
        got_T = sq.bf16_from_bits(H.host(T).view(np.uint16))
        ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref_T), 1e-30))[1] - 8)
        tol = ulp + (np.abs(Xv) @ np.abs(np.asarray(prep["L1s"], F64))) * K * 2.0 ** -24
        assert np.all(np.abs(got_T - ref_T) <= tol)


def check_y(Y, Xv, prep, bias_bits, rank, out="bf16", rows=None):
    bias = None if bias_bits is None else wl.f32_from_bf16_bits(bias_bits).astype(F64)
    Xs = Xv if rows is None else Xv[rows]
    ref = mx.forward(Xs, prep, bias, out)
    a = H.host(Y)
    if rows is not None:
        a = a[rows]
    y = a.astype(F64) if out == "f32" else sq.bf16_from_bits(a.view(np.uint16))
    assert np.all(np.isfinite(y))
    K = Xv.shape[1]
    A = np.abs(mx.dequantize_rows(ref["qx"], ref["ex"])) @ np.abs(mx.dequantize_rows(prep["qw"], prep["ew"])).T
    L = np.abs(np.asarray(ref["T"], F64)) @ np.abs(np.asarray(prep["L2"], F64))
    # T is bf16: the device's T may sit one bf16 step from the oracle's where
    # its fp32 sum straddles a rounding point (checked in check_act), which
    # moves y by up to one T step times |L2|
    T64 = np.asarray(ref["T"], F64)
    t_ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(T64), 1e-30))[1] - 8)
    LT = t_ulp @ np.abs(np.asarray(prep["L2"], F64))
    bits = 24 if out == "f32" else 8
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref["y"]), 1e-30))[1] - bits)
    tol = ulp + LT + 2.0 ** -24 * ((K // 32 + 8) * A + (rank + 8) * L)
    bad = np.abs(y - ref["y"]) > tol
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5].tolist(), y[bad][:5], ref["y"][bad][:5])
    r, c = rel_l2(y, ref["y"]), cosine(y, ref["y"])
    assert r <= 1e-3 and c >= 0.99999, (r, c)
    return r


@pytest.mark.parametrize("M,K,rank", [(64, 256, 16), (77, 320, 32), (130, 128, 0), (1, 64, 16), (200, 192, 64)])
def test_mx_quantize_act_bit_exact(M, K, rank):
    say("mx act", M, K, rank)
    Xb, Xv, prep, _ = problem(M, K, 64, rank, seed=M + K + rank, outliers=(3, K - 7))
    qx, ux, T = run_act(Xb, prep, rank)
    check_act(qx, ux, T, Xv, prep, rank)


def test_mx_quantize_act_tiny_and_zero_blocks():
    """Rows of zeros, a block of subnormal-range values (below the exact-
    quotient range, IEEE division path) and huge values."""
    M, K, rank = 20, 128, 16
    Xb, Xv, prep, _ = problem(M, K, 64, rank, seed=7)
    Xv = Xv.copy()
    Xv[2, :] = 0.0
    Xv[5, 64:96] *= 2.0 ** -120
    Xv[6, :32] = 3.0e38
    Xb = wl.bf16_bits_from_f32(Xv.astype(np.float32))
    Xv = wl.f32_from_bf16_bits(Xb).astype(F64)
    qx, ux, T = run_act(Xb, prep, rank)
    check_act(qx, ux, T, Xv, prep, rank)


@pytest.mark.parametrize("M,K,N,rank,out", [
    (64, 256, 256, 16, "f32"), (64, 256, 256, 16, "bf16"), (77, 320, 40, 32, "bf16"), (1, 64, 8, 0, "f32"),
    (130, 192, 136, 64, "bf16"), (257, 512, 264, 32, "f32"),
    # large grids with ragged token and weight tails
    (1300, 256, 12352, 32, "bf16"), (1300, 128, 12416, 16, "f32"),
])
def test_mx_linear_matches_oracle(M, K, N, rank, out):
    say("mx linear", M, K, N, rank, out)
    Xb, Xv, prep, bb = problem(M, K, N, rank, seed=M * 3 + N, outliers=(1, K // 2))
    qx, ux, T = run_act(Xb, prep, rank)
    Y = run_linear(qx, ux, T, prep, None if bb is None else bb["bits"], M, N, K, rank, out)
    r = check_y(Y, Xv, prep, None if bb is None else bb["bits"], rank, out)
    say(f"  rel-L2 {r:.2e}")


def test_mx_linear_attention_projection_full():
    """The attention-projection shape (M = 4608, K = N = 3072, rank 32):
    codes, scales and every output against the oracle."""
    case = wl.CASES["attn_proj"]
    X = wl.activations(case)
    W = wl.weight(case)
    bias = wl.bias(case)
    Xv = X["values"].astype(F64)
    say("mx full attn_proj", case.M, case.K, case.N)
    prep = mx.prepare_weights(W["values"].astype(F64), sq.channel_absmax(Xv), case.rank)
    qx, ux, T = run_act(X["bits"], prep, case.rank)
    check_act(qx, ux, T, Xv, prep, case.rank)
    Y = run_linear(qx, ux, T, prep, bias["bits"], case.M, case.N, case.K, case.rank)
    r = check_y(Y, Xv, prep, bias["bits"], case.rank)
    say(f"  rel-L2 {r:.2e}")
    # the method's accuracy against the unquantized product (reported)
    yq = sq.bf16_from_bits(H.host(Y).view(np.uint16))
    yd = Xv @ W["values"].astype(F64) + wl.f32_from_bf16_bits(bias["bits"])
    say(f"  vs X W: rel-L2 {rel_l2(yq, yd):.3e}")


def test_mx_linear_mlp_up_sampled_rows():
    case = wl.CASES["mlp_up"]
    X = wl.activations(case)
    W = wl.weight(case)
    bias = wl.bias(case)
    Xv = X["values"].astype(F64)
    say("mx mlp_up sampled", case.M, case.K, case.N)
    prep = mx.prepare_weights(W["values"].astype(F64), sq.channel_absmax(Xv), case.rank)
    qx, ux, T = run_act(X["bits"], prep, case.rank)
    Y = run_linear(qx, ux, T, prep, bias["bits"], case.M, case.N, case.K, case.rank)
    rows = np.array([0, 1, 127, 128, 2047, 4095, 4096, 4607])
    check_y(Y, Xv, prep, bias["bits"], case.rank, rows=rows)


@pytest.mark.parametrize("M,K,rank", [(64, 1024, 32), (130, 3072, 16)])
def test_mx_act_split_and_single_pass_agree(M, K, rank):
    """With its workspace the pass splits K across blocks (2 and 6 ways at
    these shapes); codes and scales are identical to the single pass and T
    is within the same bound of the oracle on both paths."""
    say("mx act split", M, K, rank)
    Xb, Xv, prep, _ = problem(M, K, 64, rank, seed=M + K, outliers=(3, K - 7))
    assert b.svdq_act_workspace_bytes(M, K, rank) > 0
    a = run_act(Xb, prep, rank, split=True)
    c = run_act(Xb, prep, rank, split=False)
    # the scale matrix's padding columns (rows M..ld) are never written
    assert np.array_equal(H.host(a[0]), H.host(c[0]))
    assert np.array_equal(H.host(a[1])[:, :M], H.host(c[1])[:, :M])
    for r in (a, c):
        check_act(*r, Xv, prep, rank)
