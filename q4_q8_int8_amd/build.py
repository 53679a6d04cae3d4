"""Build libmmq.so in-tree with hipcc for gfx950.

Usage: python q4_q8_int8_amd/build.py (run as a file: importing the package loads the library
this builds).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmmq.so")

SOURCES = ["quantize.hip", "repack.hip", "mmq_gemm.hip", "mmq_skinny.hip", "mmq_gemv.hip",
           "f16_path.hip", "f16_gemm.hip", "static_scratch.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed FP32 instructions (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the epilogue reads every S on the vector ALU, and an MFMA that
    # writes accumulation registers would cost one v_accvgpr_read per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # every loop marked "#pragma unroll" in the kernels is meant to unroll completely (the
    # GEMM's super-block loop holds register tuples indexed by the step number); the default
    # size limit for such loops is below that loop's size
    "-mllvm", "-pragma-unroll-threshold=262144",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so; that line
    # is expected and harmless, anything else is shown.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source and link libmmq.so in the package directory; returns its
    path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    tmp = tempfile.mkdtemp(prefix="mmq_build_")
    try:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            objs.append(obj)
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmds.append([HIPCC, *FLAGS, *lang, "-c",
                         os.path.join(CSRC, src), "-o", obj])
        with ThreadPoolExecutor(max_workers=min(4, len(cmds))) as ex:
            for cmd, _ in zip(cmds, ex.map(_run, cmds)):
                if verbose:
                    print(" ".join(cmd))
        out_tmp = LIB + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out_tmp])
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
