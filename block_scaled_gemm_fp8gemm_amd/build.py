"""Build ``libfp8gemm.so`` (gfx950 only) in-tree with hipcc.

Usage: ``python -m block_scaled_gemm_fp8gemm_amd.build`` (or ``build()`` from
``__graft_entry__``).  Every call recompiles all sources; objects go to
``_build/`` at the repository root and the library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp8gemm.so")

SOURCES = ["api.cpp", "quantize.hip", "gemm.hip", "grouped.hip", "transpose.hip", "gemm_fp6.hip"]
# gemm.hip is compiled once more per pair of operand formats other than e4m3 x e4m3
# and once per FP8 pair for row-major B (FP8GEMM_KN), grouped.hip once more for
# MXFP4 experts
FORMAT_UNITS = [("gemm.hip", ("FP8GEMM_FMT_A=1", "FP8GEMM_FMT_B=1"), ".e5m2_e5m2"),
                ("gemm.hip", ("FP8GEMM_FMT_A=0", "FP8GEMM_FMT_B=1"), ".e4m3_e5m2"),
                ("gemm.hip", ("FP8GEMM_FMT_A=1", "FP8GEMM_FMT_B=0"), ".e5m2_e4m3"),
                ("gemm.hip", ("FP8GEMM_FMT_A=4", "FP8GEMM_FMT_B=4"), ".e2m1_e2m1"),
                ("gemm.hip", ("FP8GEMM_KN=1",), ".kn"),
                ("gemm.hip", ("FP8GEMM_KN=1", "FP8GEMM_FMT_A=1", "FP8GEMM_FMT_B=1"), ".kn_e5m2_e5m2"),
                ("gemm.hip", ("FP8GEMM_KN=1", "FP8GEMM_FMT_A=0", "FP8GEMM_FMT_B=1"), ".kn_e4m3_e5m2"),
                ("gemm.hip", ("FP8GEMM_KN=1", "FP8GEMM_FMT_A=1", "FP8GEMM_FMT_B=0"), ".kn_e5m2_e4m3"),
                ("gemm.hip", ("FP8GEMM_KN=1", "FP8GEMM_FMT_A=4", "FP8GEMM_FMT_B=4"), ".kn_e2m1_e2m1"),
                ("grouped.hip", ("FP8GEMM_FMT_A=4", "FP8GEMM_FMT_B=4"), ".e2m1_e2m1")]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfp8gemm.so)")


def _compile(hipcc: str, src: str, defines=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc, *FLAGS, *[f"-D{d}" for d in defines], *lang, "-c", os.path.join(CSRC, src),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source for gfx950 and link the library (default libfp8gemm.so).

    ``defines`` are extra preprocessor definitions (tuning switches); ``out`` is
    the path of the shared library to write.
    """
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    tag = "" if not defines else "." + "_".join(d.replace("=", "") for d in defines)
    units = [(s, tuple(defines), tag) for s in SOURCES]
    units += [(s, tuple(defines) + d, tag + t) for s, d, t in FORMAT_UNITS]
    with cf.ThreadPoolExecutor(max_workers=min(len(units), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda u: _compile(hipcc, *u), units))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
