"""The library's host preparation (C++) against the oracle, on the CPU.

Smoothing factors, and the residual + INT4 codes + scales given the
oracle's own factors, must be bit-exact. The library's SVD differs from
LAPACK's (several factorizations are correct when singular values are close),
so it is held to the Eckart-Young bar: its rank-r error may exceed the optimum
by at most a factor (1 + 1e-3)."""

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b
from bit_quantized_linear_amd import workloads as wl
from oracle import svdquant as sq
from oracle import w8a8 as o8

F64 = np.float64


def _case(name, M=None):
    case = wl.CASES[name]
    return case, wl.activations(case, M), wl.weight(case)


@pytest.mark.parametrize("name", ["tiny"])
def test_smoothing_and_residual_bit_exact(name):
    case, X, W = _case(name)
    a = sq.channel_absmax(X["values"])
    prep = sq.prepare_weights(W["values"], a, case.rank)
    lib = b.svdq_prepare_weights(W["bits"], a, case.rank)
    assert np.array_equal(lib["s"], prep["s"])
    abi = sq.to_abi(prep)
    res = b.svdq_prepare_residual(W["bits"], abi["s"], abi["l1t"], abi["l2t"])
    assert np.array_equal(res["qw"], abi["qw"])
    assert np.array_equal(res["sw"], abi["sw"])


def test_residual_bit_exact_medium_with_heavy_columns():
    """Heavy weight columns and outlier channels (attention-projection
    generators) on a cut-down 512 x 1024 weight, rank 32."""
    case = wl.CASES["attn_proj"]
    X = wl.activations(case, 256)["values"][:, :512]
    W = wl.weight(case)
    Wv = W["values"][:512, :1024]
    Wb = W["bits"][:512, :1024]
    a = sq.channel_absmax(X)
    prep = sq.prepare_weights(Wv, a, 32)
    abi = sq.to_abi(prep)
    lib = b.svdq_prepare_weights(Wb, a, 32)
    assert np.array_equal(lib["s"], abi["s"])
    res = b.svdq_prepare_residual(Wb, abi["s"], abi["l1t"], abi["l2t"])
    assert np.array_equal(res["qw"], abi["qw"]) and np.array_equal(res["sw"], abi["sw"])


@pytest.mark.parametrize("K,N,rank", [(256, 256, 16), (512, 1024, 32), (1024, 512, 64), (256, 128, 0)])
def test_library_svd_meets_eckart_young(K, N, rank):
    case = wl.CASES["attn_proj"]
    X = wl.activations(case, 128)["values"][:, :K]
    W = wl.weight(case)
    Wv, Wb = W["values"][:K, :N], W["bits"][:K, :N]
    a = sq.channel_absmax(X)
    lib = b.svdq_prepare_weights(Wb, a, rank, want_sigma=True)
    s = lib["s"].astype(F64)
    What = s[:, None] * Wv.astype(F64)
    S = np.linalg.svd(What, compute_uv=False)
    if rank == 0:
        assert lib["l1t"].size == 0
        return
    L1 = sq.bf16_from_bits(lib["l1t"]).T
    L2 = sq.bf16_from_bits(lib["l2t"]).T
    err = np.linalg.norm(What - s[:, None] * (L1 @ L2)) ** 2
    # the stored factors are bf16: compare against the optimum plus the bf16
    # rounding of the oracle's own optimal factors
    U, S2, Vt = np.linalg.svd(What, full_matrices=False)
    L1o = sq.bf16_round((U[:, :rank] * np.sqrt(S2[:rank])) / s[:, None])
    L2o = sq.bf16_round(np.sqrt(S2[:rank])[:, None] * Vt[:rank])
    err_oracle = np.linalg.norm(What - s[:, None] * (L1o @ L2o)) ** 2
    opt = (S[rank:] ** 2).sum()
    assert err <= (1 + 1e-3) * max(opt, err_oracle)
    assert np.all(np.diff(lib["sigma"]) <= 0)
    assert np.abs(lib["sigma"][0] - S[0]) <= 1e-6 * S[0]


def test_full_rank_library_svd_reconstructs():
    rng = np.random.default_rng(4)
    K = N = 64
    Wv = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    Wb = wl.bf16_bits_from_f32(Wv)
    Wv = wl.f32_from_bf16_bits(Wb).astype(F64)
    a = np.abs(rng.standard_normal(K)).astype(np.float32) + 0.5
    lib = b.svdq_prepare_weights(Wb, a, 64, want_sigma=True)
    S = np.linalg.svd(lib["s"].astype(F64)[:, None] * Wv, compute_uv=False)
    assert np.allclose(lib["sigma"], S, rtol=1e-10, atol=0)


def test_w8a8_prepare_bit_exact():
    case = wl.CASES["tiny"]
    W = wl.weight(case)
    qw_o, sw_o = o8.prepare_weights(W["values"])
    qw_l, sw_l = b.w8a8_prepare_weights(W["bits"])
    assert sw_l == float(sw_o)
    assert np.array_equal(qw_l, o8.to_abi(qw_o))


@pytest.mark.parametrize("K,N,rank", [(64, 8, 0), (192, 40, 16), (256, 136, 32)])
def test_mx_residual_matches_the_oracle_bit_exactly(K, N, rank):
    """svdq_mx_prepare_residual (C++) == oracle/mxfp4.prepare_from_factors on
    the same smoothing and factors: E2M1 codes and E8M0 exponents, written in
    the documented container (ragged 128-row blocks for N > 128)."""
    from oracle import mxfp4 as mx
    from tests.mx_format import pack_mx_codes, pack_mx_scales, unpack_mx_codes, unpack_mx_scales

    rng = np.random.default_rng(K + N + rank)
    W = wl.random_bf16(K * 3 + N, (K, N), 0.02)
    Wv = W["values"].astype(np.float64)
    s = sq.rn32(rng.uniform(0.5, 2.0, K)).astype(np.float64)
    L1s = sq.bf16_round(rng.standard_normal((K, rank)) * 0.05)
    L2 = sq.bf16_round(rng.standard_normal((rank, N)) * 0.05)
    prep = mx.prepare_from_factors(Wv, s, L1s, L2)
    out = b.svdq_mx_prepare_residual(W["bits"], s.astype(np.float32), sq.bf16_bits(L1s.T), sq.bf16_bits(L2.T))
    assert np.array_equal(out["qw"], pack_mx_codes(prep["qw"]))
    assert np.array_equal(out["uw"], pack_mx_scales(prep["ew"]))
    assert np.array_equal(unpack_mx_codes(out["qw"], K), prep["qw"])
    assert np.array_equal(unpack_mx_scales(out["uw"], N), prep["ew"])
