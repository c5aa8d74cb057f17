"""Build libsvdq.so (HIP kernels for gfx950 + host C++) in-tree.

    python -m bit_quantized_linear_amd.build

HIP sources are compiled by hipcc for gfx950 only; host C++ sources by the
ROCm clang++. Objects go to ``_build/`` beside this file and the shared
library to ``libsvdq.so`` in this package directory. The GELU table of the
fused MLP epilogue is generated first (``gelu_table.py`` ->
``_build/gelu_table.h``).
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

if __package__:
    from . import gelu_table
else:  # run as a script
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from bit_quantized_linear_amd import gelu_table

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsvdq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANGXX = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-ffp-contract=off", "-Wall", "-Wno-unused-function"]
# packed fp32 ops are disabled for all device code (v_pk_{add,mul,fma}_f32)
HIP_FLAGS = COMMON + [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
                      "-packed-fp32-ops"]
CXX_FLAGS = COMMON + ["-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__", "-pthread"]
# per-source extras: the W4A16 kernel feeds every MFMA result straight into
# VALU arithmetic, so its MFMAs write VGPRs (no accumulation-register copies)
HIP_EXTRA = {"w4a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + p.stdout)
    return p.stdout


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    gelu_table.write(os.path.join(BUILD, "gelu_table.h"))
    jobs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        jobs.append([HIPCC] + HIP_FLAGS + ["-I", BUILD] + HIP_EXTRA.get(os.path.basename(src), []) +
                    ["-c", src, "-o", obj])
    for src in sorted(glob.glob(os.path.join(CSRC, "*.cpp"))):
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        jobs.append([CLANGXX] + CXX_FLAGS + ["-c", src, "-o", obj])
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-pthread"])
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
