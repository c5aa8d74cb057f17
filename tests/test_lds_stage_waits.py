"""The GEMMs that stage operands with direct-to-LDS loads keep each stage in
its own LDS variable so that the compiler can tell the stage being refilled
from the one being read. With the stages in one array, in a kernel with
more than one LDS variable, it put a wait for every outstanding load
(`s_waitcnt vmcnt(0)`) between a stage's refill loads and its first LDS
read, so each stage waited for loads it had just issued. This compiles the
four kernels to gfx950 assembly (host only, no GPU) and checks that no wait
that needs one of a stage's direct-to-LDS loads to have landed sits between
those loads and the next LDS read unless a barrier separates them (the
intended waits come right before the barrier that ends a stage, or the one
after the prologue).
"""

import os
import re
import shutil
import subprocess

import pytest

from bit_quantized_linear_amd import build as B

SOURCES = ["w4a4_fp6_gemm.hip", "w4a4_gemm.hip", "mx_gemm.hip", "w8a8.hip"]

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) or shutil.which("python3") is None,
                                reason="hipcc not available")


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


def _stalls(lines):
    """(line, text) of every wait on the vector-memory counter that makes an
    LDS read wait for direct-to-LDS loads of the current stage: after n such
    loads (counted since the last barrier, with no load into registers after
    them), a `vmcnt(c)` with c < n can only be passed once n - c of them have
    landed, so if an LDS read follows before the next barrier, that read
    waits for the refill (text order; the loads return in issue order)."""
    found = []
    lds_loads = 0
    wait_line = None
    for i, raw in enumerate(lines):
        line = raw.strip()
        if line.endswith(":") or line.startswith(".") and not line.startswith(".LBB"):
            continue
        if re.match(r"(buffer|global)_load\S*\s.*\blds\b", line):
            lds_loads += 1
        elif re.match(r"(buffer|global|flat)_load", line) or line.startswith("s_barrier") or \
                line.startswith("s_endpgm"):
            # a load into registers: a later wait may be for it (the epilogue's
            # low-rank operands); a barrier ends the stage
            lds_loads, wait_line = 0, None
        elif lds_loads and line.startswith("s_waitcnt"):
            m = re.search(r"vmcnt\((\d+)\)", line)
            if m and int(m.group(1)) < lds_loads:
                wait_line = (i + 1, line)
        elif line.startswith("ds_read") and wait_line is not None:
            found.append(wait_line)
            lds_loads, wait_line = 0, None
    return found


@pytest.mark.parametrize("src", SOURCES)
def test_reads_do_not_wait_for_the_refill_loads(src, tmp_path):
    lines = _assembly(src, tmp_path)
    assert any(re.match(r"\s*buffer_load\S*\s.*\blds\b", l) for l in lines), "no direct-to-LDS loads found"
    stalls = _stalls(lines)
    assert not stalls, f"{src}: LDS reads wait for in-flight refill loads at {stalls[:3]}"


def test_checker_flags_the_stalling_pattern():
    """The pattern the one-array stages produced, and the intended forms."""
    bad = ["buffer_load_dwordx4 v2, s[4:7], 0 offen lds", "s_waitcnt vmcnt(0)", "ds_read_b128 v[8:11], v3"]
    good_end = ["buffer_load_dwordx4 v2, s[4:7], 0 offen lds", "ds_read_b128 v[8:11], v3",
                "s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)", "s_barrier", "ds_read_b128 v[8:11], v3"]
    epilogue = ["buffer_load_dwordx4 v2, s[4:7], 0 offen lds", "global_load_dwordx4 v[4:7], v[0:1], off",
                "s_waitcnt vmcnt(0)", "ds_read_b128 v[8:11], v3"]
    # a partial wait after a stage's refill loads stalls the reads just the same
    partial = ["buffer_load_dwordx4 v2, s[4:7], 0 offen lds"] * 8 + ["s_waitcnt vmcnt(3)",
                                                                       "ds_read_b128 v[8:11], v3"]
    # ...while a wait that leaves all of them in flight does not
    harmless = ["buffer_load_dwordx4 v2, s[4:7], 0 offen lds"] * 4 + ["s_waitcnt vmcnt(4)",
                                                                        "ds_read_b128 v[8:11], v3"]
    assert _stalls(bad) == [(2, "s_waitcnt vmcnt(0)")]
    assert _stalls(partial) == [(9, "s_waitcnt vmcnt(3)")]
    assert _stalls(harmless) == []
    assert _stalls(good_end) == []
    assert _stalls(epilogue) == []
