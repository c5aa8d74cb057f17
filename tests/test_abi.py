"""The C-ABI library: it loads, exports every symbol its header declares, and
fails closed on bad arguments and on a non-gfx950 device -- all checked
without a GPU and without any compute call (rejected calls launch nothing)."""

import ctypes as C
import os
import re

import numpy as np
import pytest

from bit_quantized_linear_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below is rejected first
MISALIGNED = 0x10008


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_0-9]+)\s*\(", text)
    keep = [n for n in names if n.startswith(("svdq_", "w8a8_", "w4a16_"))]
    return sorted(set(keep))


def test_every_declared_symbol_is_exported():
    lib = C.CDLL(b.LIB_PATH)
    names = header_functions()
    assert len(names) >= 21
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(b.SIGNATURES), "binding and header disagree"


def test_status_strings_and_version():
    assert b.svdq_version() == 8
    for s in range(7):
        assert b.status_string(s)
    assert "unknown" in b.status_string(99)


def test_no_gpu_means_unsupported_device():
    # in a container without a GPU the capability check fails closed
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert b.svdq_check_device(0) == b.SVDQ_ERR_UNSUPPORTED_DEVICE


def test_arch_override_fails_closed_before_launch():
    lib = b.lib()
    b.svdq_debug_set_arch_override("gfx942")
    try:
        st = lib.svdq_quantize_act(FAKE, FAKE, FAKE, 16, 128, 16, 64, 0, FAKE, FAKE, FAKE, None, 0, None)
        assert st == b.SVDQ_ERR_UNSUPPORTED_DEVICE
        st = lib.svdq_w4a4_linear(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 16, 64, 128, 16, 64, 1,
                                  FAKE, b.SVDQ_BF16, None)
        assert st == b.SVDQ_ERR_UNSUPPORTED_DEVICE
        st = lib.w8a8_linear(FAKE, FAKE, 1.0, None, 16, 64, 128, FAKE, 1 << 20, FAKE, None)
        assert st == b.SVDQ_ERR_UNSUPPORTED_DEVICE
    finally:
        b.svdq_debug_set_arch_override(None)


@pytest.mark.parametrize("args,expected", [
    # (M, K, rank, group) -> status
    ((16, 100, 16, 64), b.SVDQ_ERR_UNSUPPORTED_SHAPE),   # K % 64
    ((16, 128, 16, 32), b.SVDQ_ERR_UNSUPPORTED_SHAPE),   # group != 64
    ((16, 128, 24, 64), b.SVDQ_ERR_UNSUPPORTED_SHAPE),   # rank % 16
    ((16, 128, 80, 64), b.SVDQ_ERR_UNSUPPORTED_SHAPE),   # rank > 64
    ((-1, 128, 16, 64), b.SVDQ_ERR_INVALID_ARGUMENT),    # negative M
    ((16, 0, 16, 64), b.SVDQ_ERR_INVALID_ARGUMENT),      # K == 0
])
def test_quantize_act_shape_checks(args, expected):
    M, K, rank, group = args
    st = b.lib().svdq_quantize_act(FAKE, FAKE, FAKE, M, K, rank, group, 0, FAKE, FAKE, FAKE, None, 0, None)
    assert st == expected


def test_null_and_misaligned_pointers_rejected():
    lib = b.lib()
    assert lib.svdq_quantize_act(None, FAKE, FAKE, 16, 128, 16, 64, 0, FAKE, FAKE, FAKE, None, 0, None) == \
        b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.svdq_quantize_act(MISALIGNED, FAKE, FAKE, 16, 128, 16, 64, 0, FAKE, FAKE, FAKE, None, 0, None) == \
        b.SVDQ_ERR_MISALIGNED
    assert lib.svdq_quantize_act(FAKE, FAKE, FAKE, 16, 128, 16, 64, 2, FAKE, FAKE, FAKE, None, 0, None) == \
        b.SVDQ_ERR_INVALID_ARGUMENT  # unknown container
    assert lib.svdq_w4a4_linear(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 16, 60, 128, 16, 64, 0, FAKE,
                                b.SVDQ_BF16, None) == b.SVDQ_ERR_UNSUPPORTED_SHAPE  # N % 8
    assert lib.svdq_w4a4_linear(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 16, 64, 128, 16, 64, 0, FAKE,
                                7, None) == b.SVDQ_ERR_INVALID_ARGUMENT  # dtype
    assert lib.svdq_w4a4_linear(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 16, 64, 128, 16, 64, 5, FAKE,
                                b.SVDQ_BF16, None) == b.SVDQ_ERR_INVALID_ARGUMENT  # container
    assert lib.svdq_w4a4_linear(FAKE, FAKE, None, FAKE, FAKE, FAKE, None, 16, 64, 128, 16, 64, 1, FAKE,
                                b.SVDQ_BF16, None) == b.SVDQ_ERR_INVALID_ARGUMENT  # T missing
    assert lib.w8a8_linear(FAKE, FAKE, 1.0, None, 16, 64, 128, FAKE, 16, FAKE, None) == \
        b.SVDQ_ERR_INVALID_ARGUMENT  # workspace too small
    assert lib.w8a8_linear(FAKE, FAKE, float("nan"), None, 16, 64, 128, FAKE, 1 << 20, FAKE, None) == \
        b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.w8a8_linear(FAKE, FAKE, 1.0, None, 16, 64, 133184, FAKE, 1 << 40, FAKE, None) == \
        b.SVDQ_ERR_UNSUPPORTED_SHAPE  # K 127^2 overflows int32
    assert lib.svdq_debug_group_partials(FAKE, FAKE, 16, 64, 96, 64, 0, FAKE, None) == \
        b.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert lib.svdq_channel_absmax(FAKE, 4, 12, FAKE, None) == b.SVDQ_ERR_UNSUPPORTED_SHAPE


def test_workspace_size_covers_codes():
    assert b.w8a8_workspace_bytes(4608, 3072) >= 4608 * 3072 + b.w8a8_workspace_offset_codes()
    assert b.w8a8_workspace_bytes(-1, 64) == 0


def test_host_prepare_rejects_bad_input():
    W = np.zeros((128, 64), np.uint16)
    a = np.ones(128, np.float32)
    with pytest.raises(b.SvdqError) as e:
        b.svdq_prepare_weights(W[:100], a[:100], 16)
    assert e.value.status == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    with pytest.raises(b.SvdqError) as e:
        b.svdq_prepare_weights(W, a, 80)
    assert e.value.status == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    Wn = W.copy()
    Wn[3, 5] = 0x7FC0  # NaN
    with pytest.raises(b.SvdqError) as e:
        b.svdq_prepare_weights(Wn, a, 16)
    assert e.value.status == b.SVDQ_ERR_NUMERICAL
    a2 = a.copy()
    a2[0] = np.inf
    with pytest.raises(b.SvdqError) as e:
        b.svdq_prepare_weights(W, a2, 16)
    assert e.value.status == b.SVDQ_ERR_NUMERICAL


def test_row_bytes_of_the_containers():
    assert b.svdq_qrow_bytes(3072, b.QFMT_INT4) == 1536
    assert b.svdq_qrow_bytes(3072, b.QFMT_FP6) == 2304
    assert b.svdq_qrow_bytes(100, b.QFMT_FP6) == 0
    assert b.svdq_qrow_bytes(128, 9) == 0


def test_repack_to_fp6_matches_the_documented_layout():
    """The library's host repack vs the test-side FP6 writer built from the
    header's description of the container (bit-exact)."""
    from oracle import svdquant as sq
    from tests.fp6_format import pack_fp6, unpack_fp6

    rng = np.random.default_rng(12)
    codes = rng.integers(-7, 8, (37, 320)).astype(np.int8)
    codes[0, :] = 7
    codes[1, :] = -7
    codes[2, :] = 0
    packed = sq.pack_int4(codes)
    fp6 = b.svdq_repack_codes(packed, 320, b.QFMT_FP6)
    assert np.array_equal(fp6, pack_fp6(codes))
    assert np.array_equal(unpack_fp6(fp6, 320), codes)
    assert np.array_equal(b.svdq_repack_codes(packed, 320, b.QFMT_INT4), packed)
    bad = packed.copy()
    bad[3, 0] = 0x08  # a nibble holding -8
    with pytest.raises(b.SvdqError) as e:
        b.svdq_repack_codes(bad, 320, b.QFMT_FP6)
    assert e.value.status == b.SVDQ_ERR_NUMERICAL


@pytest.mark.parametrize("rows,K", [(1, 64), (127, 128), (128, 192), (129, 320), (300, 384)])
def test_fp6_container_blocks_of_128_rows(rows, K):
    """Ragged row counts: library repack == test-side writer, and one code
    lands where the header's formula puts it (block b at 128 b (3K/4), group
    g of the block at + g n_b 48, row r at + 48 r, plane 0 byte 0)."""
    from oracle import svdquant as sq
    from tests.fp6_format import pack_fp6

    rng = np.random.default_rng(rows * 1000 + K)
    codes = rng.integers(-7, 8, (rows, K)).astype(np.int8)
    fp6 = b.svdq_repack_codes(sq.pack_int4(codes), K, b.QFMT_FP6)
    assert np.array_equal(fp6, pack_fp6(codes))
    m, g = rows - 1, K // 64 - 1
    one = np.zeros((rows, K), np.int8)
    one[m, g * 64] = 3  # code 3 -> FP6 bits 0b000011 at bit 0 of H_0
    flat = b.svdq_repack_codes(sq.pack_int4(one), K, b.QFMT_FP6).reshape(-1)
    b0 = (m // 128) * 128
    nb = min(128, rows - b0)
    pos = b0 * (K // 4 * 3) + g * nb * 48 + (m - b0) * 48
    assert flat[pos] == 3 and np.count_nonzero(flat) == 1


@pytest.mark.parametrize("K,N", [(64, 1), (128, 16), (192, 40), (320, 33), (1024, 96)])
def test_w4a16_container_matches_the_oracle_and_the_documented_layout(K, N):
    """Library W4A16 preparation == the oracle's codes and scales written by
    the test-side writer of the header's layout (bit-exact), including odd
    group counts and ragged column counts (padding u = 8, scale 0)."""
    from oracle import w4a16 as o16
    from tests.w4a16_format import pack_w4a16, unpack_w4a16
    from bit_quantized_linear_amd import workloads as wl

    rng = np.random.default_rng(K * 7 + N)
    Wv = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    Wv[:, 0] *= 8
    if N > 2:
        Wv[64:128, 2] = 0.0  # an all-zero group
    Wb = wl.bf16_bits_from_f32(Wv)
    Wf = wl.f32_from_bf16_bits(Wb)
    qw, sw = o16.prepare_weights(Wf)
    lib_buf = b.w4a16_prepare_weights(Wb)
    assert lib_buf.size == b.w4a16_weight_bytes(K, N) == (N + 31) // 32 * ((K // 64 + 1) // 2) * 2304
    assert np.array_equal(lib_buf, pack_w4a16(qw, sw))
    q2, s2 = unpack_w4a16(lib_buf, K, N)
    assert np.array_equal(q2, qw) and np.array_equal(s2, sw)


def test_w4a16_one_code_lands_where_the_header_says():
    from tests.w4a16_format import UNIT
    from bit_quantized_linear_amd import workloads as wl

    K, N = 256, 72
    W = np.zeros((K, N), np.float32)
    # group 3 -> pair p = 1, d = 2 (group 2p + 1, first half) + 1 (second half): d = 3;
    # column 32 b + 16 j + c with b = 2, j = 0, c = 7; slot l = 16 * 2 + 7 (k slot 2), i = 5
    k, n = 64 * 3 + 32 + 8 * 2 + 5, 32 * 2 + 7
    W[k, n] = 1.75  # scale 0.25, code 7 -> u = 15
    buf = b.w4a16_prepare_weights(wl.bf16_bits_from_f32(W))
    P = 2
    unit = buf[(2 * P + 1) * UNIT:(2 * P + 2) * UNIT]
    word = int(unit[:1024].view(np.uint32)[(16 * 2 + 7) * 4 + 3])
    assert (word >> (16 + 4 * 2)) & 0xF == 15  # i = 5 -> bits 16 + 4*2
    assert word & ~(0xF << 24) == 0x88888888 & ~(0xF << 24)
    assert unit[2048:].view(np.float32)[(16 * 7 + 8 * 0 + 4 * 1) // 4] == 0.25  # c = 7, j = 0, e = 1
    assert np.count_nonzero(unit[2048:].view(np.float32)) == 1


def test_w4a16_shape_and_argument_checks():
    lib = b.lib()
    assert b.w4a16_weight_bytes(100, 8) == 0 and b.w4a16_weight_bytes(64, 0) == 0
    with pytest.raises(b.SvdqError) as e:
        b.w4a16_prepare_weights(np.zeros((100, 8), np.uint16))
    assert e.value.status == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    Wn = np.zeros((64, 8), np.uint16)
    Wn[1, 1] = 0x7F80  # inf
    with pytest.raises(b.SvdqError) as e:
        b.w4a16_prepare_weights(Wn)
    assert e.value.status == b.SVDQ_ERR_NUMERICAL
    assert lib.w4a16_linear(FAKE, FAKE, None, 2, 16, 100, 64, FAKE, None) == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert lib.w4a16_linear(FAKE, FAKE, None, 2, 16, 128, 32, FAKE, None) == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert lib.w4a16_linear(FAKE, FAKE, None, 1, 16, 28736, 64, FAKE, None) == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert lib.w4a16_linear(FAKE, None, None, 2, 16, 128, 64, FAKE, None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.w4a16_linear(FAKE, FAKE, None, 2, 0, 128, 64, FAKE, None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.w4a16_linear(MISALIGNED, FAKE, None, 2, 16, 128, 64, FAKE, None) == b.SVDQ_ERR_MISALIGNED
    assert lib.w4a16_linear(FAKE, FAKE, None, 1 << 20, 16, 1 << 11, 64, FAKE, None) == \
        b.SVDQ_ERR_UNSUPPORTED_SHAPE  # M K 2 bytes past 32-bit offsets
    b.svdq_debug_set_arch_override("gfx942")
    try:
        assert lib.w4a16_linear(FAKE, FAKE, None, 2, 16, 128, 64, FAKE, None) == b.SVDQ_ERR_UNSUPPORTED_DEVICE
    finally:
        b.svdq_debug_set_arch_override(None)


def _mlp(M=16, N=128, K=128, rank=16, rank_down=16, ws=1 << 20, **kw):
    a = dict(qx=FAKE, sx=FAKE, T=FAKE, qw=FAKE, sw=FAKE, l2t=FAKE, bias=None, smooth=FAKE, l1t=FAKE, qxd=FAKE,
             sxd=FAKE, Td=FAKE, yup=None, work=FAKE)
    a.update(kw)
    return b.lib().svdq_w4a4_linear_gelu_quantize(
        a["qx"], a["sx"], a["T"], a["qw"], a["sw"], a["l2t"], a["bias"], M, N, K, rank, 64, a["smooth"], a["l1t"],
        rank_down, a["qxd"], a["sxd"], a["Td"], a["yup"], a["work"], ws, None)


def test_mlp_pair_entry_point_fails_closed():
    assert b.svdq_mlp_workspace_bytes(4608, 12288, 32) == 96 * 4608 * 32 * 4
    assert b.svdq_mlp_workspace_bytes(4608, 12288, 0) == 0
    assert b.svdq_mlp_workspace_bytes(-1, 128, 16) == 0
    assert _mlp(N=96) == b.SVDQ_ERR_UNSUPPORTED_SHAPE          # the down-projection's K % 64
    assert _mlp(rank_down=8) == b.SVDQ_ERR_UNSUPPORTED_SHAPE   # rank_down % 16
    assert _mlp(rank_down=80) == b.SVDQ_ERR_UNSUPPORTED_SHAPE  # rank_down > 64
    assert _mlp(K=100) == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert _mlp(ws=16) == b.SVDQ_ERR_INVALID_ARGUMENT          # workspace too small
    assert _mlp(work=None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert _mlp(smooth=None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert _mlp(Td=None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert _mlp(qxd=MISALIGNED) == b.SVDQ_ERR_MISALIGNED
    assert _mlp(yup=MISALIGNED) == b.SVDQ_ERR_MISALIGNED
    assert _mlp(M=-1) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert b.lib().svdq_debug_gelu_bf16(None, FAKE, 4, None) == b.SVDQ_ERR_INVALID_ARGUMENT
    b.svdq_debug_set_arch_override("gfx942")
    try:
        assert _mlp() == b.SVDQ_ERR_UNSUPPORTED_DEVICE
        assert _mlp(rank_down=0, ws=0, work=None, l1t=None, Td=None) == b.SVDQ_ERR_UNSUPPORTED_DEVICE
        assert b.lib().svdq_debug_gelu_bf16(FAKE, FAKE, 4, None) == b.SVDQ_ERR_UNSUPPORTED_DEVICE
    finally:
        b.svdq_debug_set_arch_override(None)


def test_act_workspace_is_optional_but_checked():
    lib = b.lib()
    need = b.svdq_act_workspace_bytes(4608, 3072, 32)
    assert need == 8 * 4608 * 32 * 4  # K split eight ways at this shape
    assert b.svdq_act_workspace_bytes(4608, 12288, 32) == 28 * 4608 * 32 * 4
    assert b.svdq_act_workspace_bytes(4608, 3072, 0) == 0
    assert b.svdq_act_workspace_bytes(4608, 100, 32) == 0
    args = (FAKE, FAKE, FAKE, 4608, 3072, 32, 64, 1, FAKE, FAKE, FAKE)
    assert lib.svdq_quantize_act(*args, FAKE, need - 4, None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.svdq_quantize_act(*args, MISALIGNED, need, None) == b.SVDQ_ERR_MISALIGNED
    assert lib.svdq_mx_quantize_act(FAKE, FAKE, FAKE, 4608, 3072, 32, FAKE, FAKE, FAKE, FAKE, 16, None) == \
        b.SVDQ_ERR_INVALID_ARGUMENT


def test_noalloc_scratch_covers_every_split():
    """The fixed 32 MiB scratch of svdq_quantize_act_noalloc holds T's fp32
    partials for every shape: the split into p parts keeps p * M <= 131072,
    so p * M * rank * 4 <= 131072 * 64 * 4 bytes."""
    worst = 0
    for M in list(range(1, 33000, 61)) + [4608, 16383, 16384, 16385, 32760, 32768, 65536, 131072, 262144]:
        for K in (64, 512, 1024, 3072, 4096, 5120, 12288, 16384, 65536):
            worst = max(worst, b.svdq_act_workspace_bytes(M, K, 64))
    assert 0 < worst <= 32 << 20


def test_noalloc_entry_point_fails_closed():
    lib = b.lib()
    args = lambda M, K, rank, group, qfmt, X=FAKE: (X, FAKE, FAKE, M, K, rank, group, qfmt, FAKE, FAKE, FAKE, None)
    assert lib.svdq_quantize_act_noalloc(*args(16, 100, 16, 64, 1)) == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert lib.svdq_quantize_act_noalloc(*args(16, 128, 24, 64, 1)) == b.SVDQ_ERR_UNSUPPORTED_SHAPE
    assert lib.svdq_quantize_act_noalloc(*args(16, 128, 16, 64, 3)) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.svdq_quantize_act_noalloc(*args(16, 128, 16, 64, 1, X=None)) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.svdq_quantize_act_noalloc(*args(16, 128, 16, 64, 1, X=MISALIGNED)) == b.SVDQ_ERR_MISALIGNED
    b.svdq_debug_set_arch_override("gfx942")
    try:
        assert lib.svdq_quantize_act_noalloc(*args(4608, 3072, 32, 64, 1)) == b.SVDQ_ERR_UNSUPPORTED_DEVICE
    finally:
        b.svdq_debug_set_arch_override(None)


def test_mfma_rate_probe_counts_and_fails_closed():
    # 2 M N K per MFMA, 4 chains, 4 waves per block
    assert b.svdq_debug_mfma_ops(0, 3, 5) == 2 * 32 * 32 * 64 * 4 * 4 * 3 * 5
    assert b.svdq_debug_mfma_ops(1, 1, 1) == 2 * 32 * 32 * 32 * 4 * 4
    assert b.svdq_debug_mfma_ops(2, 1, 1) == 2 * 32 * 32 * 16 * 4 * 4
    assert b.svdq_debug_mfma_ops(3, 1, 1) == 0 and b.svdq_debug_mfma_ops(0, 0, 1) == 0
    lib = b.lib()
    assert lib.svdq_debug_mfma_rate(3, 4, 10, FAKE, None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.svdq_debug_mfma_rate(0, 4, 10, None, None) == b.SVDQ_ERR_INVALID_ARGUMENT
    assert lib.svdq_debug_mfma_rate(0, 4, 10, MISALIGNED, None) == b.SVDQ_ERR_MISALIGNED
