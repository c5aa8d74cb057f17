"""The FP6 code packing (`pack_fp6_16` in quant_common.h) converts two
16-value operands with gfx950's v_cvt_scalef32_2xpk16_fp6_f32 but defines
only their first 8 values each (the rest are left undefined and only feed the
result's unused upper dwords). When the compiler put the 6-register result
on top of defined operand values (v[16:21] over the second operand
v[14:29], so the result's first register was that operand's third value),
the instruction packed a 0 for that value. The helper keeps both operands
live across the conversion; this compiles the kernels that pack codes to
gfx950 assembly (host only, no GPU) and checks every conversion: its result
registers overlap no register that holds one of the first 8 values of
either operand.
"""

import os
import re
import shutil
import subprocess

import pytest

from bit_quantized_linear_amd import build as B

SOURCES = ["act_quant.hip", "w4a4_fp6_gemm.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) or shutil.which("python3") is None,
                                reason="hipcc not available")

CVT = re.compile(r"v_cvt_scalef32_2xpk16_fp6_f32\s+v\[(\d+):(\d+)\],\s*v\[(\d+):(\d+)\],\s*v\[(\d+):(\d+)\]")


def _assembly(src, tmp_path):
    os.makedirs(B.BUILD, exist_ok=True)
    from bit_quantized_linear_amd import gelu_table
    header = os.path.join(B.BUILD, "gelu_table.h")
    if not os.path.exists(header):
        gelu_table.write(header)
    out = tmp_path / (src + ".s")
    subprocess.run([B.HIPCC] + B.HIP_FLAGS + ["-I", B.CSRC, "-I", B.BUILD, "--cuda-device-only", "-S",
                    os.path.join(B.CSRC, src), "-o", str(out)], check=True, capture_output=True)
    return out.read_text().splitlines()


def overlaps(line):
    """Registers of the conversion's result that hold a defined operand value
    (the first 8 registers of either 16-register operand), or None when the
    line is not such a conversion."""
    m = CVT.search(line)
    if not m:
        return None
    d0, d1, a0, a1, b0, b1 = map(int, m.groups())
    assert d1 - d0 == 5 and a1 - a0 == 15 and b1 - b0 == 15, line
    dst = set(range(d0, d1 + 1))
    used = set(range(a0, a0 + 8)) | set(range(b0, b0 + 8))
    return sorted(dst & used)


def test_checker_flags_an_overlapping_result():
    assert overlaps("v_cvt_scalef32_2xpk16_fp6_f32 v[16:21], v[38:53], v[14:29], 1.0") == [16, 17, 18, 19, 20, 21]
    assert overlaps("v_cvt_scalef32_2xpk16_fp6_f32 v[0:5], v[0:15], v[16:31], 1.0") == [0, 1, 2, 3, 4, 5]
    # on the undefined upper halves only: allowed
    assert overlaps("v_cvt_scalef32_2xpk16_fp6_f32 v[8:13], v[0:15], v[16:31], 1.0") == []
    assert overlaps("v_cvt_scalef32_2xpk16_fp6_f32 v[32:37], v[24:39], v[16:31], 1.0") == []
    assert overlaps("v_mfma_f32_32x32x1_2b_f32 v[0:31], v1, v2, 0") is None


@pytest.mark.parametrize("src", SOURCES)
def test_packing_result_never_overlaps_defined_operands(src, tmp_path):
    lines = _assembly(src, tmp_path)
    found = [(i, l.strip()) for i, l in enumerate(lines) if overlaps(l) is not None]
    assert found, f"{src}: no FP6 packing conversion found"
    bad = [(i, l) for i, l in found if overlaps(l)]
    assert not bad, bad[:5]
