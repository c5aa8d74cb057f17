"""The library's GELU table (generated at build time by
bit_quantized_linear_amd/gelu_table.py from the C library's float64 erfc)
against the oracle's GELU, on every one of its 3328 entries (no GPU)."""

import numpy as np

from bit_quantized_linear_amd import gelu_table
from oracle import mlp
from oracle import svdquant as sq


def test_table_equals_the_oracle_on_every_entry():
    t = np.array(gelu_table.table(), dtype=np.uint16)
    assert t.size == gelu_table.ENTRIES == 3328
    idx = np.arange(t.size)
    sign, rest = idx // 1664, idx % 1664
    bits = ((sign << 15) | ((rest // 128 + gelu_table.EXP_LO) << 7) | (rest % 128)).astype(np.uint16)
    want = sq.bf16_bits(mlp.gelu_bf16(sq.bf16_from_bits(bits)))
    assert np.array_equal(t, want)


def test_built_header_holds_the_table():
    import os

    from bit_quantized_linear_amd import build

    path = os.path.join(build.BUILD, "gelu_table.h")
    if not os.path.exists(path):
        import pytest

        pytest.skip("library not built")
    text = open(path).read()
    vals = [int(v, 16) for v in text.split("= {")[1].split("}")[0].replace("\n", " ").split(",")]
    assert vals == gelu_table.table()
