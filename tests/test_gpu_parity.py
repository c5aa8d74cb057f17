"""HIP path vs the CPU oracle, through the C-ABI (needs an MI355X).

Bars: packed INT4 codes, INT8 codes, group scales and int32 partials /
accumulators bit-exact; T within one bf16 ulp per element and rel-L2 <= 1e-3;
outputs within an a-priori per-element bound of fp32 rounding plus one output
ulp (tests/parity_bounds.py), and overall rel-L2 <= 1e-3, cosine >= 0.99999
and all finite. Inputs are prepared by the oracle (or, for the chain the
bench runs, by the library's own preparation, whose factors the oracle then
takes) and handed to the library; nothing the device computes flows into
the oracle's arithmetic.
"""

import functools

import sys

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b
from bit_quantized_linear_amd import workloads as wl
from oracle import mlp
from oracle import svdquant as sq
from oracle import w8a8 as o8
from tests import gpu_harness as H
from tests import parity_bounds as PB
from tests.oracle_pins import cosine, rel_l2

pytestmark = pytest.mark.gpu

F64 = np.float64
REL_L2 = 1e-3
COS = 0.99999


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert b.svdq_check_device(torch.cuda.current_device()) == b.SVDQ_OK, "not a gfx950 device"


def check_T(T_gpu, T_ref, X=None, L1s=None):
    """T within one bf16 ulp of the oracle plus the worst-case error of an fp32
    sum of K products (K 2^-24 sum |x l|), per element; rel-L2 <= 1e-3."""
    Th = T_gpu if isinstance(T_gpu, np.ndarray) else H.host(T_gpu)
    got = sq.bf16_from_bits(Th.view(np.uint16))
    ref = np.asarray(T_ref, dtype=F64)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-30))[1] - 8)
    tol = ulp
    if X is not None:
        A = np.abs(np.asarray(X, dtype=F64)) @ np.abs(np.asarray(L1s, dtype=F64))
        tol = ulp + A * (np.asarray(X).shape[1] * 2.0 ** -24)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5].tolist(), got[bad][:5], ref[bad][:5])
    assert rel_l2(got, ref) <= REL_L2
    return got


def check_output(y, ref):
    assert np.all(np.isfinite(y))
    assert rel_l2(y, ref) <= REL_L2, rel_l2(y, ref)
    assert cosine(y, ref) >= COS, cosine(y, ref)


def check_w4a4(y, ref, prep, bias, out, T_dev=None, cols=slice(None), what="w4a4"):
    """A W4A4 output y [M, N'] against the oracle's forward `ref` (its qx, sx,
    T and rounded y) on weights `prep`, restricted to output columns `cols`:
    every element within the a-priori bound, then the overall bars. T_dev is
    the device's T (float values) when the device computed its own."""
    qw = np.asarray(prep["qw"])[:, cols]
    sw = np.asarray(prep["sw"])[:, cols]
    L2 = np.asarray(prep["L2"])[:, cols] if np.asarray(prep["L2"]).size else None
    bv = None if bias is None else np.asarray(bias)[cols]
    ry = np.asarray(ref["y"])[:, cols]
    dT = None if T_dev is None else np.asarray(T_dev, dtype=F64) - np.asarray(ref["T"], dtype=F64)
    tol = PB.w4a4_tolerance(ref["qx"], ref["sx"], qw, sw, ref["T"] if L2 is not None else None, L2, bv, y, ry,
                            out, dT)
    PB.check_elementwise(y, ry, tol, what)
    check_output(y, ry)


def T_values(T):
    Th = T if isinstance(T, np.ndarray) else H.host(T)
    return sq.bf16_from_bits(Th.view(np.uint16))


# ------------------------------------------------------------ act quant --

@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
@pytest.mark.parametrize("M,K,rank", [(64, 1024, 32), (130, 3072, 16), (300, 512, 0)])
def test_quantize_act_split_and_single_pass_agree(M, K, rank, qfmt):
    """With its workspace the pass splits K across blocks; codes and scales
    are identical to the single pass, and T is within the same bound of the
    oracle on both paths (the split changes only T's fp32 summation order)."""
    say("quantize_act split", M, K, rank, qfmt)
    p = H.make_problem(M, K, 64, rank, seed=M + 1, outliers=(3, K - 5))
    a = H.run_quantize_act(p["X"]["bits"], p["abi"], rank, qfmt, split=True)
    c = H.run_quantize_act(p["X"]["bits"], p["abi"], rank, qfmt, split=False)
    cx, csx = sq.quantize_activations(p["X"]["values"], p["prep"]["s"])
    for r in (a, c):
        assert np.array_equal(H.host(r[0]), H.pack_codes(cx, qfmt))
        assert np.array_equal(H.host(r[1]), csx)
        if rank:
            check_T(r[2], sq.lowrank_down(p["X"]["values"], p["prep"]["L1s"]), p["X"]["values"], p["prep"]["L1s"])


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
@pytest.mark.parametrize("shape", [(64, 256, 16), (77, 320, 32), (1, 64, 16), (130, 128, 0), (33, 192, 64)])
def test_quantize_act_small(shape, qfmt):
    M, K, rank = shape
    say("quantize_act", shape, qfmt)
    p = H.make_problem(M, K, max(rank, 16) * 2 if rank else 64, rank, seed=M, outliers=(3, K - 5),
                       zero_rows=(0,) if M > 2 else ())
    qx, sx, T = H.run_quantize_act(p["X"]["bits"], p["abi"], rank, qfmt)
    cx, csx = sq.quantize_activations(p["X"]["values"], p["prep"]["s"])
    assert np.array_equal(H.host(qx), H.pack_codes(cx, qfmt))
    assert np.array_equal(H.host(sx), csx)
    if rank:
        check_T(T, sq.lowrank_down(p["X"]["values"], p["prep"]["L1s"]), p["X"]["values"], p["prep"]["L1s"])


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_quantize_act_attention_projection_full(qfmt):
    case, X, W, bias, prep, abi = H.prepared_case("attn_proj")
    say("quantize_act attn_proj", X["bits"].shape, qfmt)
    qx, sx, T = H.run_quantize_act(X["bits"], abi, case.rank, qfmt)
    cx, csx = sq.quantize_activations(X["values"], prep["s"])
    assert np.array_equal(H.host(qx), H.pack_codes(cx, qfmt))
    assert np.array_equal(H.host(sx), csx)
    check_T(T, sq.lowrank_down(X["values"], prep["L1s"]), X["values"], prep["L1s"])


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
@pytest.mark.parametrize("order", ["shuffled", "by_magnitude"])
def test_quantize_act_every_bf16_value(order, qfmt):
    """Every bf16 bit pattern whose quotient by the smoothing factor stays
    finite (signed zeros, subnormals, normals up to 2^121) goes through the
    smoothing divide, the group absmax and the code rounding once: codes and
    scales bit-exact against the oracle's IEEE fp32 divisions. Shuffled, a
    group mixes all magnitudes; ordered by magnitude, a group holds 64
    neighbouring magnitudes and its codes cover the whole grid."""
    say("quantize_act every bf16 value", order, qfmt)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) < 0xF8
    bits = np.where(finite, bits, np.uint16(0)).astype(np.uint16)
    rng = np.random.default_rng(65536)
    if order == "shuffled":
        bits = rng.permutation(bits)
    else:
        bits = bits[np.argsort(bits & np.uint16(0x7FFF), kind="stable")]
    bits = bits.reshape(512, 128)
    vals = wl.f32_from_bf16_bits(bits)
    s = rng.uniform(1.0 / 16, 16.0, size=128).astype(np.float32)
    qx, sx, _ = H.run_quantize_act(bits, {"s": s}, 0, qfmt)
    cx, csx = sq.quantize_activations(vals, s)
    assert np.array_equal(H.host(sx), csx)
    assert np.array_equal(H.host(qx), H.pack_codes(cx, qfmt))


def test_channel_absmax_matches_oracle():
    t = H.torch()
    say("channel_absmax")
    case = wl.CASES["attn_proj"]
    X = wl.activations(case, 1000)
    am = t.zeros(case.K, dtype=t.float32, device="cuda")
    b.svdq_channel_absmax(H.dev(X["bits"][:600]), am)
    b.svdq_channel_absmax(H.dev(X["bits"][600:]), am)  # running max over two batches
    t.cuda.synchronize()
    assert np.array_equal(H.host(am), sq.channel_absmax(X["values"]))


# ----------------------------------------------------------- partials ---

@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
@pytest.mark.parametrize("shape", [(64, 256, 256), (100, 192, 136), (130, 128, 264), (300, 384, 520)])
def test_group_partials_bit_exact(shape, qfmt):
    M, K, N = shape
    say("partials", shape, qfmt)
    t = H.torch()
    rng = np.random.default_rng(M + K + N)
    cx = rng.integers(-7, 8, (M, K)).astype(np.int8)
    cw = rng.integers(-7, 8, (K, N)).astype(np.int8)
    cx[0, :64] = 7
    cw[:64, 0] = 7  # the largest partial, 64 * 49
    cx[1, :64] = -7
    P = t.empty((K // 64, M, N), dtype=t.int32, device="cuda")
    b.svdq_debug_group_partials(H.dev(H.pack_codes(cx, qfmt)), H.dev(H.pack_codes(cw.T, qfmt)), P, M, N, K,
                                qfmt=qfmt)
    t.cuda.synchronize()
    ref = sq.group_partials(cx, cw)
    assert np.array_equal(H.host(P).astype(np.int64), ref)
    assert ref[0, 0, 0] == 64 * 49 and ref[0, 1, 0] == -64 * 49


# -------------------------------------------------------------- linear ---

@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_w4a4_linear_tiny(out, qfmt):
    case, X, W, bias, prep, abi = H.prepared_case("tiny")
    say("linear tiny", out, qfmt)
    M, K, N, r = case.M, case.K, case.N, case.rank
    qwb = H.weights_bytes(prep, abi, qfmt)
    qx, sx, T = H.run_quantize_act(X["bits"], abi, r, qfmt)
    Y = H.run_linear(qx, sx, T, abi, bias["bits"], M, N, K, r, out, qfmt, qwb)
    ref = sq.forward(X["values"], prep, bias["values"], out)
    check_w4a4(H.y_values(Y, out), ref, prep, bias["values"], out, T_values(T))
    # the GEMM alone on the oracle's own codes, scales and T
    Y2 = H.run_linear(H.dev(H.pack_codes(ref["qx"], qfmt)), H.dev(ref["sx"]), H.dev(sq.bf16_bits(ref["T"])),
                      abi, bias["bits"], M, N, K, r, out, qfmt, qwb)
    check_w4a4(H.y_values(Y2, out), ref, prep, bias["values"], out)


# The FP6 GEMM runs 128 x 64 block tiles when they spread the work over the
# CUs markedly better than 128 x 128 ones: small shapes take the 64-row
# tiles; (200, 128, 32768, 16), whose 512 tiles of 128 x 128 fill the 256
# CUs exactly twice, keeps the 128-row tiles with a ragged last row tile.
@pytest.mark.parametrize("shape", [(77, 320, 200, 16), (1, 64, 16, 16), (257, 512, 136, 32), (130, 256, 264, 0),
                                   (65, 128, 384, 64), (300, 256, 520, 32), (200, 128, 32768, 16)])
@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_w4a4_linear_ragged(shape, qfmt):
    M, K, N, r = shape
    say("linear ragged", shape, qfmt)
    p = H.make_problem(M, K, N, r, seed=N, outliers=(1,), zero_rows=(M - 1,) if M > 1 else ())
    qx, sx, T = H.run_quantize_act(p["X"]["bits"], p["abi"], r, qfmt)
    Y = H.run_linear(qx, sx, T, p["abi"], p["bias"]["bits"], M, N, K, r, "f32", qfmt,
                     H.weights_bytes(p["prep"], p["abi"], qfmt))
    ref = sq.forward(p["X"]["values"], p["prep"], p["bias"]["values"], "f32")
    check_w4a4(H.y_values(Y, "f32"), ref, p["prep"], p["bias"]["values"], "f32", T_values(T) if r else None)


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_w4a4_linear_no_bias_zero_rows(qfmt):
    M, K, N, r = 40, 128, 64, 16
    say("linear no bias", qfmt)
    p = H.make_problem(M, K, N, r, seed=5, bias=False, zero_rows=(0, 7, 39))
    qx, sx, T = H.run_quantize_act(p["X"]["bits"], p["abi"], r, qfmt)
    Y = H.run_linear(qx, sx, T, p["abi"], None, M, N, K, r, "f32", qfmt, H.weights_bytes(p["prep"], p["abi"], qfmt))
    ref = sq.forward(p["X"]["values"], p["prep"], None, "f32")
    y = H.y_values(Y, "f32")
    check_w4a4(y, ref, p["prep"], None, "f32", T_values(T))
    assert np.all(y[[0, 7, 39]] == 0.0)


# The two containers hold the same codes, and their kernels apply the same
# arithmetic in the same order (the INT4 one on 256 times each partial, which
# a power-of-two factor leaves exact in fp32 while the accumulator is a
# normal number), so their outputs agree byte for byte. The shapes take both
# FP6 tile heights and both scale-load paths of each kernel (token counts
# that are and are not multiples of 4).
@pytest.mark.parametrize("shape", [(77, 320, 200, 16), (300, 256, 520, 32), (260, 3072, 3072, 32),
                                   (200, 128, 32768, 16), (1023, 256, 8192, 16)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_containers_give_identical_outputs(shape, out):
    M, K, N, r = shape
    say("containers agree", shape, out)
    p = H.make_problem(M, K, N, r, seed=M + N, outliers=(1,), zero_rows=(M - 1,))
    ys = []
    for qfmt in H.FORMATS:
        qx, sx, T = H.run_quantize_act(p["X"]["bits"], p["abi"], r, qfmt)
        Y = H.run_linear(qx, sx, T, p["abi"], p["bias"]["bits"], M, N, K, r, out, qfmt,
                         H.weights_bytes(p["prep"], p["abi"], qfmt))
        ys.append(H.host(Y).view(np.uint8))
    assert np.array_equal(ys[0], ys[1])


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_w4a4_attention_projection_full(qfmt):
    case, X, W, bias, prep, abi = H.prepared_case("attn_proj")
    M, K, N, r = case.M, case.K, case.N, case.rank
    say("linear attn_proj full", (M, K, N, r), qfmt)
    qx, sx, T = H.run_quantize_act(X["bits"], abi, r, qfmt)
    Y = H.run_linear(qx, sx, T, abi, bias["bits"], M, N, K, r, "bf16", qfmt, H.weights_bytes(prep, abi, qfmt))
    ref = sq.forward(X["values"], prep, bias["values"], "bf16")
    check_w4a4(H.y_values(Y, "bf16"), ref, prep, bias["values"], "bf16", T_values(T))
    # the quality of the method itself is reported, not gated
    say("  rel-L2 vs unquantized X W + b:",
        rel_l2(ref["y64"], X["values"].astype(F64) @ W["values"].astype(F64) + bias["values"]))


# the oracle's preparation of a full-size case (40 s for the video case),
# shared by the tests of both containers and the one-GPU share below
prepared_full = functools.lru_cache(maxsize=1)(H.prepared_case)


@functools.lru_cache(maxsize=1)
def full_reference(name):
    """The oracle's whole forward of a named full-size case (main product in
    its dense closed form), shared by the tests of both containers."""
    case, X, W, bias, prep, abi = prepared_full(name)
    say("  oracle forward", name, (case.M, case.K, case.N))
    return sq.forward_dense(X["values"], prep, bias["values"], "bf16")


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
@pytest.mark.parametrize("name", ["mlp_up", "video"])
def test_w4a4_full_size_every_row(name, qfmt):
    """Full-size shapes in the launch configuration the bench times (the
    activation pass with its workspace, then the GEMM): every code, scale and
    T element, and every output element against the oracle's whole forward."""
    case, X, W, bias, prep, abi = prepared_full(name)
    M, K, N, r = case.M, case.K, case.N, case.rank
    say("linear full-size", name, (M, K, N, r), qfmt)
    qx, sx, T = H.run_quantize_act(X["bits"], abi, r, qfmt)
    Y = H.run_linear(qx, sx, T, abi, bias["bits"], M, N, K, r, "bf16", qfmt, H.weights_bytes(prep, abi, qfmt))
    ref = full_reference(name)
    assert np.array_equal(H.unpack_codes(H.host(qx), K, qfmt), ref["qx"])
    assert np.array_equal(H.host(sx), ref["sx"])
    Tv = check_T(T, ref["T"], X["values"], prep["L1s"])
    y = sq.bf16_from_bits(H.host(Y).view(np.uint16))
    del Y
    check_w4a4(y, ref, prep, bias["values"], "bf16", Tv, what=f"{name} {qfmt}")


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_w4a4_video_one_gpu_share(qfmt):
    """One GPU's share of the video linear under token (row) parallelism over
    8 GPUs: the first 4095 of its 32760 tokens (15 * 256 + 255 rows, a ragged
    last row tile) through the weights prepared for the whole workload, with
    the activation pass's workspace as the bench launches it; every code,
    scale and T element and every output element against the oracle."""
    case, X, W, bias, prep, abi = prepared_full("video")
    M, K, N, r = 4095, case.K, case.N, case.rank
    say("linear one GPU's share of video", (M, K, N, r), qfmt)
    Xb = np.ascontiguousarray(X["bits"][:M])
    Xv = X["values"][:M]
    qx, sx, T = H.run_quantize_act(Xb, abi, r, qfmt)
    Y = H.run_linear(qx, sx, T, abi, bias["bits"], M, N, K, r, "bf16", qfmt, H.weights_bytes(prep, abi, qfmt))
    ref = sq.forward_dense(Xv, prep, bias["values"], "bf16")
    assert np.array_equal(H.unpack_codes(H.host(qx), K, qfmt), ref["qx"])
    assert np.array_equal(H.host(sx), ref["sx"])
    Tv = check_T(T, ref["T"], Xv, prep["L1s"])
    y = sq.bf16_from_bits(H.host(Y).view(np.uint16))
    check_w4a4(y, ref, prep, bias["values"], "bf16", Tv, what=f"video share {qfmt}")


def test_library_prepared_chain_mlp_up():
    """The route the bench runs, from raw weights: the calibration statistic
    on the device, the library's host preparation (smoothing, its own SVD,
    bf16 factors, residual codes and scales), the FP6 repack, the activation
    pass and the GEMM -- against the oracle evaluated on the library's own
    smoothing factors and low-rank factors (several SVD results are correct,
    so the factors are the one thing taken over; reading R19). The library's
    s, codes and scales must equal the oracle's for those factors, and every
    output element must be within the bound of the oracle's forward."""
    t = H.torch()
    case = wl.CASES["mlp_up"]
    M, K, N, r = case.M, case.K, case.N, case.rank
    say("library-prepared chain", (M, K, N, r))
    X, W, bias = wl.activations(case), wl.weight(case), wl.bias(case)
    Xd = H.dev(X["bits"])
    amax = t.zeros(K, dtype=t.float32, device="cuda")
    b.svdq_channel_absmax(Xd, amax)
    t.cuda.synchronize()
    amax_h = H.host(amax)
    assert np.array_equal(amax_h, sq.channel_absmax(X["values"]))
    lib = b.svdq_prepare_weights(W["bits"], amax_h, r, want_sigma=True)
    s_or = sq.smoothing_factors(amax_h, W["values"])
    assert np.array_equal(lib["s"], s_or)
    L1s = sq.bf16_from_bits(lib["l1t"]).T
    L2 = sq.bf16_from_bits(lib["l2t"]).T
    prep = sq.prepare_from_factors(W["values"], lib["s"], L1s, L2)
    assert np.array_equal(sq.unpack_int4(lib["qw"]).T, prep["qw"])
    assert np.array_equal(lib["sw"], prep["sw"])
    # the factors are a rank-r approximation of the smoothed weight as good as
    # the best one (Eckart-Young, bar of reading R19)
    _, S, _ = sq.smoothed_svd(W["values"], s_or)
    err2 = np.linalg.norm(s_or[:, None].astype(F64) * W["values"] - (s_or[:, None] * L1s) @ L2) ** 2
    assert err2 <= (1 + 1e-2) * np.sum(S[r:] ** 2)
    qw6 = H.dev(b.svdq_repack_codes(lib["qw"], K, b.QFMT_FP6))
    abi = {"s": lib["s"], "l1t": lib["l1t"], "l2t": lib["l2t"], "sw": lib["sw"]}
    qx, sx, T = H.run_quantize_act(X["bits"], abi, r, b.QFMT_FP6)
    Yd = t.empty((M, N), dtype=t.int16, device="cuda")
    b.svdq_w4a4_linear(qx, sx, T, qw6, H.dev(lib["sw"]), H.dev(lib["l2t"]), H.dev(bias["bits"]), Yd, M, N, K, r,
                       qfmt=b.QFMT_FP6)
    t.cuda.synchronize()
    ref = sq.forward_dense(X["values"], prep, bias["values"], "bf16")
    assert np.array_equal(H.unpack_codes(H.host(qx), K, b.QFMT_FP6), ref["qx"])
    assert np.array_equal(H.host(sx), ref["sx"])
    Tv = check_T(T, ref["T"], X["values"], L1s)
    y = sq.bf16_from_bits(H.host(Yd).view(np.uint16))
    check_w4a4(y, ref, prep, bias["values"], "bf16", Tv, what="library-prepared mlp_up")


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_w4a4_tiny_magnitude_groups(qfmt):
    """Rows and single groups of X scaled far down (2^-100 .. 2^-120): the
    activation pass takes its IEEE-division branch, the scale products
    sx sw fall into fp32's subnormal range, and the GEMM must still apply
    them; fp32 output, no bias, every element within the bound."""
    M, K, N, r = 96, 256, 136, 16
    say("tiny-magnitude groups", qfmt)
    p = H.make_problem(M, K, N, r, seed=21, bias=False, outliers=(9,))
    Xv = p["X"]["values"].astype(np.float32).copy()
    Xv[5] *= np.float32(2.0 ** -100)
    Xv[6] *= np.float32(2.0 ** -120)
    Xv[7, 64:128] *= np.float32(2.0 ** -110)
    Xv[90, :64] *= np.float32(2.0 ** -126)
    bits = wl.bf16_bits_from_f32(Xv)
    Xv = wl.f32_from_bf16_bits(bits)
    qx, sx, T = H.run_quantize_act(bits, p["abi"], r, qfmt)
    Y = H.run_linear(qx, sx, T, p["abi"], None, M, N, K, r, "f32", qfmt, H.weights_bytes(p["prep"], p["abi"], qfmt))
    ref = sq.forward(Xv, p["prep"], None, "f32")
    assert np.array_equal(H.unpack_codes(H.host(qx), K, qfmt), ref["qx"])
    assert np.array_equal(H.host(sx), ref["sx"])
    prod = ref["sx"][:, 6][:, None].astype(F64) * p["prep"]["sw"].astype(F64)
    assert np.any((prod > 0) & (prod < 2.0 ** -126)), "no subnormal scale product exercised"
    Tv = T_values(T)
    y = H.y_values(Y, "f32")
    check_w4a4(y, ref, p["prep"], None, "f32", Tv, what="tiny groups")
    # the scaled rows themselves, on their own scale
    for row in (5, 6, 7, 90):
        assert np.any(y[row] != 0.0)
        assert rel_l2(y[row], ref["y"][row]) <= REL_L2, row


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_w4a4_mlp_down_projection_sampled(qfmt):
    """The MLP pair's second projection: input = GELU of the oracle's
    up-projection output (on the host), K = 12288."""
    case, X, W, bias, prep, abi = H.prepared_case("mlp_up")
    say("linear mlp_down", qfmt)
    rows = np.arange(0, 640)  # five full row tiles of 128
    up = sq.forward(X["values"][rows], prep, bias["values"], "bf16")
    gv = mlp.gelu_bf16(up["y"])
    G = {"bits": sq.bf16_bits(gv), "values": gv}
    Wd = wl.mlp_down_weight()
    bd = wl.mlp_down_bias()
    a = sq.channel_absmax(G["values"])
    prep_d = sq.prepare_weights(Wd["values"], a, 32)
    abi_d = sq.to_abi(prep_d)
    M, K, N = len(rows), wl.MLP_DOWN.K, wl.MLP_DOWN.N
    qx, sx, T = H.run_quantize_act(G["bits"], abi_d, 32, qfmt)
    Y = H.run_linear(qx, sx, T, abi_d, bd["bits"], M, N, K, 32, "bf16", qfmt, H.weights_bytes(prep_d, abi_d, qfmt))
    ref = sq.forward(G["values"], prep_d, bd["values"], "bf16")
    assert np.array_equal(H.host(qx), H.pack_codes(ref["qx"], qfmt))
    check_w4a4(H.y_values(Y, "bf16"), ref, prep_d, bd["values"], "bf16", T_values(T))


# -------------------------------------------------------- metamorphic ---

@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
@pytest.mark.parametrize("r", [0, 16])
def test_power_of_two_scaling_and_negation(r, qfmt):
    """X -> 4X: identical codes, scales x4 and outputs x4 bit-exactly (every
    rounding commutes with a power-of-two scale). X -> -X: negated codes and
    equal scales; the outputs negate exactly on the integer path (r = 0) and
    to within 1e-6 relative when the bf16 MFMAs of the low-rank branch
    (whose internal accumulation rounding is the hardware's) take part."""
    M, K, N = 96, 256, 128
    say("metamorphic", r, qfmt)
    p = H.make_problem(M, K, N, r, seed=3, bias=False)
    qwb = H.weights_bytes(p["prep"], p["abi"], qfmt)
    Xv = p["X"]["values"].astype(np.float32)
    outs = {}
    for tag, f in (("x1", 1.0), ("x4", 4.0), ("neg", -1.0)):
        bits = wl.bf16_bits_from_f32(Xv * np.float32(f))
        qx, sx, T = H.run_quantize_act(bits, p["abi"], r, qfmt)
        Y = H.run_linear(qx, sx, T, p["abi"], None, M, N, K, r, "f32", qfmt, qwb)
        outs[tag] = (H.host(qx), H.host(sx), H.host(T) if r else None, H.y_values(Y, "f32"))
    cx1 = H.unpack_codes(outs["x1"][0], K, qfmt)
    assert np.array_equal(outs["x4"][0], outs["x1"][0])
    assert np.array_equal(outs["x4"][1], outs["x1"][1] * 4)
    assert np.array_equal(outs["x4"][3], outs["x1"][3] * 4)
    assert np.array_equal(H.unpack_codes(outs["neg"][0], K, qfmt), -cx1)
    assert np.array_equal(outs["neg"][1], outs["x1"][1])
    if r == 0:
        assert np.array_equal(outs["neg"][3], -outs["x1"][3])
    else:
        tn = sq.bf16_from_bits(outs["neg"][2].view(np.uint16))
        t1 = sq.bf16_from_bits(outs["x1"][2].view(np.uint16))
        say("  T exact negation:", bool(np.array_equal(tn, -t1)), "max |T(-X) + T(X)|:", float(np.abs(tn + t1).max()))
        d = outs["neg"][3] + outs["x1"][3]
        say("  Y exact negation:", bool(not d.any()), "max |Y(-X) + Y(X)|:", float(np.abs(d).max()))
        assert rel_l2(outs["neg"][3], -outs["x1"][3]) <= 1e-6


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_run_to_run_byte_identical(qfmt):
    case, X, W, bias, prep, abi = H.prepared_case("tiny")
    say("determinism", qfmt)
    M, K, N, r = case.M, case.K, case.N, case.rank
    qwb = H.weights_bytes(prep, abi, qfmt)
    res = []
    for _ in range(3):
        qx, sx, T = H.run_quantize_act(X["bits"], abi, r, qfmt)
        Y = H.run_linear(qx, sx, T, abi, bias["bits"], M, N, K, r, "bf16", qfmt, qwb)
        res.append((H.host(qx).tobytes(), H.host(sx).tobytes(), H.host(T).tobytes(), H.host(Y).tobytes()))
    assert res[0] == res[1] == res[2]


@pytest.mark.parametrize("qfmt", H.FORMATS, ids=H.FORMAT_IDS)
def test_one_activation_pass_feeds_several_projections(qfmt):
    """Shared-input projections (attention Q, K and V): the smoothing comes
    from the concatenated weight, one svdq_quantize_act feeds the GEMM of
    each projection (its column slice of the prepared weight, packed on its
    own) and the GEMM of the concatenation; all match the oracle of the
    concatenated linear."""
    M, K, Np, r = 200, 512, 136, 16
    say("shared activation pass, three projections", (M, K, Np, r), qfmt)
    p = H.make_problem(M, K, 3 * Np, r, seed=33, outliers=(5, 77))
    prep, abi = p["prep"], p["abi"]
    qx, sx, T = H.run_quantize_act(p["X"]["bits"], abi, r, qfmt)
    ref = sq.forward(p["X"]["values"], prep, p["bias"]["values"], "bf16")
    bias_bits = p["bias"]["bits"]
    qw_codes = np.asarray(prep["qw"]).T  # [N, K]
    for j in range(3):
        cols = slice(j * Np, (j + 1) * Np)
        part = {"sw": np.ascontiguousarray(abi["sw"][:, cols]), "l2t": np.ascontiguousarray(abi["l2t"][cols]),
                "qw": np.ascontiguousarray(abi["qw"][cols])}
        qw_j = H.pack_codes(qw_codes[cols], qfmt)
        Y = H.run_linear(qx, sx, T, part, np.ascontiguousarray(bias_bits[cols]), M, Np, K, r, "bf16", qfmt, qw_j)
        check_w4a4(H.y_values(Y, "bf16"), ref, prep, p["bias"]["values"], "bf16", T_values(T), cols=cols)
    Yall = H.run_linear(qx, sx, T, abi, bias_bits, M, 3 * Np, K, r, "bf16", qfmt, H.weights_bytes(prep, abi, qfmt))
    check_w4a4(H.y_values(Yall, "bf16"), ref, prep, p["bias"]["values"], "bf16", T_values(T))


def test_empty_batch_is_a_no_op():
    t = H.torch()
    say("M = 0")
    K, N, r = 128, 64, 16
    p = H.make_problem(8, K, N, r, seed=9)
    e16 = t.empty((0, K), dtype=t.int16, device="cuda")
    qx = t.empty((0, K // 2), dtype=t.uint8, device="cuda")
    sx = t.empty((K // 64, 0), dtype=t.float32, device="cuda")
    T = t.empty((0, r), dtype=t.int16, device="cuda")
    b.svdq_quantize_act(e16, H.dev(p["abi"]["s"]), H.dev(p["abi"]["l1t"]), qx, sx, T, r)
    Y = t.empty((0, N), dtype=t.int16, device="cuda")
    b.svdq_w4a4_linear(qx, sx, T, H.dev(p["abi"]["qw"]), H.dev(p["abi"]["sw"]), H.dev(p["abi"]["l2t"]),
                       None, Y, 0, N, K, r)
    t.cuda.synchronize()


# ---------------------------------------------------------------- W8A8 ---

# K = 576 is five 128-byte stages, the last one half (the GEMM runs stages
# in pairs and the odd one after them)
@pytest.mark.parametrize("shape", [(64, 256, 256), (77, 192, 136), (1, 64, 8), (200, 576, 264)])
def test_w8a8_small(shape):
    M, K, N = shape
    say("w8a8", shape)
    X = wl.random_bf16(M * 7 + K, (M, K))
    Xv = X["values"].copy()
    Xv[:, 2] *= 10
    Xb = wl.bf16_bits_from_f32(Xv)
    Xv = wl.f32_from_bf16_bits(Xb)
    W = wl.random_bf16(N + 1, (K, N), 0.02)
    bias = wl.random_bf16(N + 2, (N,), 0.01)
    qw, sw = o8.prepare_weights(W["values"])
    Y, codes, scale = H.w8a8_run(Xb, o8.to_abi(qw), float(sw), bias["bits"])
    ref = o8.forward(Xv, qw, sw, bias["values"])
    assert scale == float(ref["sx"])
    assert np.array_equal(codes, ref["qx"])
    check_w8a8(H.y_values(Y, "bf16"), ref, sw, bias["values"])


def check_w8a8(y, ref, sw, bias, what="w8a8"):
    tol = PB.w8a8_tolerance(ref["acc"], ref["sx"], sw, bias, y, ref["y"])
    PB.check_elementwise(y, ref["y"], tol, what)
    check_output(y, ref["y"])


@pytest.mark.parametrize("name", ["w8a8_attn", "video_w8a8"])
def test_w8a8_full_shapes(name):
    """The W8A8 linear on its attention shape (4608 x 3072 x 3072) and on the
    video shape (32760 x 5120 x 5120, the same shapes as the video W4A4
    linear): the tensor scale and every int8 code of X bit-exact, every
    output element within the bound."""
    case = wl.CASES[name]
    say("w8a8 full", name, (case.M, case.K, case.N))
    X = wl.activations(case)
    W = wl.weight(case)
    bias = wl.bias(case)
    qw, sw = o8.prepare_weights(W["values"])
    Y, codes, scale = H.w8a8_run(X["bits"], o8.to_abi(qw), float(sw), bias["bits"])
    ref = o8.forward(X["values"], qw, sw, bias["values"])
    assert scale == float(ref["sx"])
    assert np.array_equal(codes, ref["qx"])
    del codes
    check_w8a8(H.y_values(Y, "bf16"), ref, sw, bias["values"], name)


@pytest.mark.parametrize("shape", [(64, 256, 256), (130, 320, 136), (200, 576, 264)])
def test_w8a8_accumulators_bit_exact(shape):
    M, K, N = shape
    say("w8a8 acc", shape)
    t = H.torch()
    rng = np.random.default_rng(K)
    qx = rng.integers(-127, 128, (M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, (K, N)).astype(np.int8)
    qx[0, :] = 127
    qw[:, 0] = 127
    acc = t.empty((M, N), dtype=t.int32, device="cuda")
    b.w8a8_debug_acc(H.dev(qx), H.dev(o8.to_abi(qw)), acc, M, N, K)
    t.cuda.synchronize()
    ref = o8.accumulate(qx, qw)
    assert np.array_equal(H.host(acc).astype(np.int64), ref)
    assert ref[0, 0] == K * 127 * 127
