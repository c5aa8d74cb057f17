"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin fails for each: the pins are only worth something if they catch the
errors they were chosen for."""

import numpy as np
import pytest

from oracle import svdquant as sq
from tests import test_oracle_svdquant as pins

F64 = np.float64

_orig_quantize_rows = sq.quantize_int4_rows
_orig_residual = sq.residual
_orig_lowrank = sq.lowrank_factors
_orig_main = sq.main_product
_orig_bf16 = sq.bf16_round
_orig_linear = sq.linear_from_parts


def _mut_absmax_over_8(V, group=64):
    old = sq.QMAX
    try:
        sq.QMAX = 8
        return _orig_quantize_rows(V, group)
    finally:
        sq.QMAX = old


def _mut_round_half_away(V, group=64):
    V = np.asarray(V, dtype=np.float32)
    rows, K = V.shape
    Vg = V.reshape(rows, K // group, group).astype(F64)
    amax = np.max(np.abs(Vg), axis=2)
    scale = sq.rn32(amax / 7)
    safe = np.where(scale > 0, scale.astype(F64), 1.0)
    quot = sq.rn32(Vg / safe[:, :, None]).astype(F64)
    codes = np.clip(np.sign(quot) * np.floor(np.abs(quot) + 0.5), -7, 7)
    codes = np.where(scale[:, :, None] > 0, codes, 0)
    return codes.reshape(rows, K).astype(np.int8), scale


def _mut_residual_plus(W, s, L1s, L2):
    D = sq.lowrank_product(L1s, L2)
    return sq.rn32(np.asarray(s, F64)[:, None] * (np.asarray(W, F64) + D))


def _mut_no_inverse_smoothing(W, s, rank, round_to_bf16=True):
    U, S, Vt = sq.smoothed_svd(W, s)
    root = np.sqrt(S[:rank])
    L1s = U[:, :rank] * root[None, :]
    L2 = root[:, None] * Vt[:rank, :]
    if round_to_bf16:
        L1s, L2 = sq.bf16_round(L1s), sq.bf16_round(L2)
    return L1s, L2, S


def _mut_swapped_uv(W, s, rank, round_to_bf16=True):
    U, S, Vt = sq.smoothed_svd(W, s)
    root = np.sqrt(S[:rank])
    # wrong: take the right singular vectors for the K side
    L1s = (Vt[:rank, :].T * root[None, :]) / np.asarray(s, F64)[:, None]
    L2 = root[:, None] * U[:, :rank].T
    if round_to_bf16:
        L1s, L2 = sq.bf16_round(L1s), sq.bf16_round(L2)
    return L1s, L2, S


def _mut_group_off_by_one(qx, sx, qw, sw, group=64):
    sx = np.asarray(sx)
    return _orig_main(qx, np.roll(sx, 1, axis=0), qw, sw, group)


def _mut_scale_not_applied_to_weight(qx, sx, qw, sw, group=64):
    return _orig_main(qx, sx, qw, np.ones_like(np.asarray(sw)), group)


def _mut_truncating_bf16(x):
    x = np.asarray(x, dtype=F64)
    out = x.copy()
    nz = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[nz])
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    out[nz] = np.trunc(x[nz] / q) * q
    return out


def _mut_drop_bias(qx, sx, T, qw, sw, L2, bias=None, group=64):
    return _orig_linear(qx, sx, T, qw, sw, L2, None, group)


def _mut_drop_lowrank(qx, sx, T, qw, sw, L2, bias=None, group=64):
    return _orig_linear(qx, sx, None, qw, sw, L2, bias, group)


MUTANTS = {
    "absmax/8": ("quantize_int4_rows", _mut_absmax_over_8),
    "round-half-away": ("quantize_int4_rows", _mut_round_half_away),
    "residual W+D": ("residual", _mut_residual_plus),
    "1/s not folded": ("lowrank_factors", _mut_no_inverse_smoothing),
    "U/V swapped": ("lowrank_factors", _mut_swapped_uv),
    "group scale off by one": ("main_product", _mut_group_off_by_one),
    "weight scale dropped": ("main_product", _mut_scale_not_applied_to_weight),
    "bf16 truncation": ("bf16_round", _mut_truncating_bf16),
    "bias dropped": ("linear_from_parts", _mut_drop_bias),
    "low-rank dropped": ("linear_from_parts", _mut_drop_lowrank),
}

PIN_TESTS = [
    pins.test_bf16_round_matches_exact_rational_rounding,
    pins.test_golden_int4_group_rounding,
    pins.test_golden_w4a4_tiny,
    lambda: pins.test_brute_force_whole_pipeline("f32"),
    pins.test_main_product_equals_dequantize_then_matmul,
    pins.test_full_rank_identity,
    pins.test_on_grid_inputs_are_exact,
    pins.test_eckart_young_error_of_the_factors,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(sq, attr, fn)
    caught = []
    for t in PIN_TESTS:
        try:
            t()
        except (AssertionError, ValueError):
            caught.append(getattr(t, "__name__", "lambda"))
    assert caught, f"no pin caught the planted mistake '{name}'"
