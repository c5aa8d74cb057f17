"""The MLP pair on the device (svdq_w4a4_linear_gelu_quantize): HIP path vs
the CPU oracle, through the C-ABI (needs an MI355X).

Stage-wise, as for the standalone passes: the fused kernel's bf16 y_up is
byte-identical to svdq_w4a4_linear's output on the same operands and within
the per-element bound of the oracle's up-projection; from that y_up, the
oracle's GELU and activation quantizer give the down-projection's codes and
group scales bit-exactly and T within one bf16 ulp plus the bound of an fp32
sum; the down-projection run on the fused outputs is within the per-element
bound of the oracle's down-projection of the same GELU output, and matches
the oracle's whole pair overall (rel-L2 <= 1e-3, cosine >= 0.99999). The
device's GELU rule is checked on every bf16 input.
"""

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b
from bit_quantized_linear_amd import workloads as wl
from oracle import mlp
from oracle import svdquant as sq
from tests import gpu_harness as H
from tests.fp6_format import pack_fp6
from tests.test_gpu_parity import T_values, check_output, check_T, check_w4a4

pytestmark = pytest.mark.gpu

FP6 = b.QFMT_FP6


def say(*a):
    print(*a, flush=True)


def test_device_gelu_on_every_bf16_input():
    say("gelu every bf16")
    t = H.torch()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    y = H.dev(bits)
    g = t.empty_like(y)
    b.svdq_debug_gelu_bf16(y, g)
    t.cuda.synchronize()
    got = sq.bf16_from_bits(H.host(g).view(np.uint16))
    with np.errstate(invalid="ignore"):
        want = mlp.gelu_bf16(sq.bf16_from_bits(bits))
    same = ((got == want) & (np.signbit(got) == np.signbit(want))) | (np.isnan(got) & np.isnan(want))
    assert same.all(), bits[~same][:10]


def test_device_gelu_tails_and_unaligned_views():
    """The elementwise pass on lengths that are not a multiple of its 8-value
    vectors, and on views that are not 16-byte aligned (one value at a time)."""
    t = H.torch()
    bits = (np.arange(70001, dtype=np.uint32) * 2654435761 % 65536).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        want = mlp.gelu_bf16(sq.bf16_from_bits(bits))
    y = H.dev(bits)
    for lo, hi in ((0, 70001), (0, 8197), (1, 70001), (3, 1000)):
        say("gelu view", lo, hi)
        g = t.zeros(70001, dtype=t.int16, device="cuda")
        b.svdq_debug_gelu_bf16(y[lo:hi], g[lo:hi])
        t.cuda.synchronize()
        got = sq.bf16_from_bits(H.host(g).view(np.uint16)[lo:hi])
        w = want[lo:hi]
        same = ((got == w) & (np.signbit(got) == np.signbit(w))) | (np.isnan(got) & np.isnan(w))
        assert same.all()
        assert not H.host(g)[:lo].any() and not H.host(g)[hi:].any()


def pair_problem(M, K, N, N2, rank, rank_down, seed):
    """Up-projection [K -> N] on seeded X, down-projection [N -> N2] whose
    smoothing is calibrated on the oracle's GELU of the up output."""
    p = H.make_problem(M, K, N, rank, seed=seed, outliers=(3, K - 5), zero_rows=(0,) if M > 2 else ())
    up = sq.forward(p["X"]["values"], p["prep"], p["bias"]["values"], "bf16")
    g = mlp.gelu_bf16(up["y"])
    Wd = wl.random_bf16(seed * 10 + 7, (N, N2), 0.02)
    bd = wl.random_bf16(seed * 10 + 8, (N2,), 0.01)
    prep_d = sq.prepare_weights(Wd["values"], sq.channel_absmax(g), rank_down)
    return p, prep_d, sq.to_abi(prep_d), bd


def run_fused(Xbits, abi, prep, bias_bits, abi_d, M, N, K, rank, rank_down, with_y=True):
    t = H.torch()
    qx, sx, T = H.run_quantize_act(Xbits, abi, rank, FP6)
    qw6 = H.dev(H.weights_bytes(prep, abi, FP6))
    qxd = t.empty((M, b.svdq_qrow_bytes(N, FP6)), dtype=t.uint8, device="cuda")
    sxd = t.empty((N // 64, M), dtype=t.float32, device="cuda")
    Td = t.empty((M, rank_down), dtype=t.int16, device="cuda") if rank_down else None
    yup = t.empty((M, N), dtype=t.int16, device="cuda") if with_y else None
    wsb = b.svdq_mlp_workspace_bytes(M, N, rank_down)
    ws = t.empty(wsb, dtype=t.uint8, device="cuda") if wsb else None
    b.svdq_w4a4_linear_gelu_quantize(qx, sx, T, qw6, H.dev(abi["sw"]), H.dev(abi["l2t"]) if rank else None,
                                     H.dev(bias_bits) if bias_bits is not None else None, M, N, K, rank,
                                     H.dev(abi_d["s"]), H.dev(abi_d["l1t"]) if rank_down else None, rank_down,
                                     qxd, sxd, Td, yup, ws)
    t.cuda.synchronize()
    return {"qx": qx, "sx": sx, "T": T, "qw6": qw6, "qxd": qxd, "sxd": sxd, "Td": Td, "yup": yup}


@pytest.mark.parametrize("M,K,N,N2,rank,rank_down", [
    (64, 256, 128, 64, 16, 16), (77, 128, 192, 64, 0, 32), (130, 192, 320, 128, 32, 64),
    (1, 64, 64, 64, 16, 0), (257, 256, 256, 64, 32, 16),
])
def test_fused_up_projection_emits_the_down_projections_inputs(M, K, N, N2, rank, rank_down):
    say("mlp pair", M, K, N, N2, rank, rank_down)
    p, prep_d, abi_d, bd = pair_problem(M, K, N, N2, rank, rank_down, seed=M + N)
    r = run_fused(p["X"]["bits"], p["abi"], p["prep"], p["bias"]["bits"], abi_d, M, N, K, rank, rank_down)
    # y_up: the same kernel's main loop and rounding as svdq_w4a4_linear
    Y = H.run_linear(r["qx"], r["sx"], r["T"], p["abi"], p["bias"]["bits"], M, N, K, rank, "bf16", FP6,
                     H.weights_bytes(p["prep"], p["abi"], FP6))
    yup_bits = H.host(r["yup"]).view(np.uint16)
    assert np.array_equal(yup_bits, H.host(Y).view(np.uint16))
    y_up = sq.bf16_from_bits(yup_bits)
    up = sq.forward(p["X"]["values"], p["prep"], p["bias"]["values"], "bf16")
    check_w4a4(y_up, up, p["prep"], p["bias"]["values"], "bf16", T_values(r["T"]) if rank else None, what="y_up")
    # the down-projection's activation side from the device's own y_up
    side = mlp.down_activation_side(y_up, prep_d)
    assert np.array_equal(H.host(r["qxd"]), pack_fp6(side["qx"]))
    assert np.array_equal(H.host(r["sxd"]), side["sx"])
    if rank_down:
        check_T(r["Td"], side["T"], side["g"], prep_d["L1s"])
    # the fused outputs drive the down-projection: per element against the
    # oracle's down-projection of the same g, and the whole pair overall
    Yd = H.run_linear(r["qxd"], r["sxd"], r["Td"], abi_d, bd["bits"], M, N2, N, rank_down, "bf16", FP6,
                      H.weights_bytes(prep_d, abi_d, FP6))
    yd = H.y_values(Yd, "bf16")
    down = sq.forward(side["g"], prep_d, bd["values"], "bf16")
    check_w4a4(yd, down, prep_d, bd["values"], "bf16", T_values(r["Td"]) if rank_down else None, what="y_down")
    ref = mlp.forward(p["X"]["values"], p["prep"], p["bias"]["values"], prep_d, bd["values"])
    check_output(yd, ref["y_down"])


def test_fused_outputs_do_not_depend_on_y_up_being_written():
    M, K, N, N2, rank, rank_down = 96, 128, 256, 64, 16, 32
    say("mlp pair without y_up")
    p, prep_d, abi_d, _ = pair_problem(M, K, N, N2, rank, rank_down, seed=11)
    a = run_fused(p["X"]["bits"], p["abi"], p["prep"], p["bias"]["bits"], abi_d, M, N, K, rank, rank_down)
    c = run_fused(p["X"]["bits"], p["abi"], p["prep"], p["bias"]["bits"], abi_d, M, N, K, rank, rank_down,
                  with_y=False)
    for key in ("qxd", "sxd", "Td"):
        assert np.array_equal(H.host(a[key]), H.host(c[key])), key


def test_fused_mlp_up_full_shape_every_row():
    """C4 at full size (M 4608, K 3072, N 12288, ranks 32), in the launch
    configuration the bench times, checked stage-wise on every row: y_up per
    element against the oracle's up-projection; the down-projection's codes,
    scales and T against the oracle's activation side of the device's y_up;
    the down-projection run on them per element against the oracle's
    down-projection of the same g."""
    case, X, W, bias, prep, abi = H.prepared_case("mlp_up")
    M, K, N = case.M, case.K, case.N
    say("mlp pair full", M, K, N)
    up = sq.forward_dense(X["values"], prep, bias["values"], "bf16")
    g = mlp.gelu_bf16(up["y"])
    Wd, bd = wl.mlp_down_weight(), wl.mlp_down_bias()
    prep_d = sq.prepare_weights(Wd["values"], sq.channel_absmax(g), 32)
    del g
    abi_d = sq.to_abi(prep_d)
    r = run_fused(X["bits"], abi, prep, bias["bits"], abi_d, M, N, K, 32, 32)
    y_up = sq.bf16_from_bits(H.host(r["yup"]).view(np.uint16))
    check_w4a4(y_up, up, prep, bias["values"], "bf16", T_values(r["T"]), what="y_up full")
    del up
    side = mlp.down_activation_side(y_up, prep_d)
    assert np.array_equal(H.unpack_codes(H.host(r["qxd"]), N, FP6), side["qx"])
    assert np.array_equal(H.host(r["sxd"]), side["sx"])
    Td = check_T(r["Td"], side["T"], side["g"], prep_d["L1s"])
    N2 = wl.MLP_DOWN.N
    Yd = H.run_linear(r["qxd"], r["sxd"], r["Td"], abi_d, bd["bits"], M, N2, N, 32, "bf16", FP6,
                      H.weights_bytes(prep_d, abi_d, FP6))
    down = sq.forward_dense(side["g"], prep_d, bd["values"], "bf16")
    check_w4a4(H.y_values(Yd, "bf16"), down, prep_d, bd["values"], "bf16", Td, what="y_down full")


def test_fused_pair_without_bias_and_deterministic():
    """No up-projection bias; two runs give identical bytes."""
    M, K, N, N2, rank, rank_down = 150, 192, 384, 64, 16, 32
    say("mlp pair no bias")
    p, prep_d, abi_d, _ = pair_problem(M, K, N, N2, rank, rank_down, seed=23)
    a = run_fused(p["X"]["bits"], p["abi"], p["prep"], None, abi_d, M, N, K, rank, rank_down)
    c = run_fused(p["X"]["bits"], p["abi"], p["prep"], None, abi_d, M, N, K, rank, rank_down)
    for key in ("qxd", "sxd", "Td", "yup"):
        assert np.array_equal(H.host(a[key]), H.host(c[key])), key
    y_up = sq.bf16_from_bits(H.host(a["yup"]).view(np.uint16))
    check_w4a4(y_up, sq.forward(p["X"]["values"], p["prep"], None, "bf16"), p["prep"], None, "bf16",
               T_values(a["T"]), what="y_up no bias")
    side = mlp.down_activation_side(y_up, prep_d)
    assert np.array_equal(H.host(a["qxd"]), pack_fp6(side["qx"]))
    assert np.array_equal(H.host(a["sxd"]), side["sx"])
    check_T(a["Td"], side["T"], side["g"], prep_d["L1s"])
