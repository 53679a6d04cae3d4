"""The kernels that use the direct-to-LDS load helper leave M0 to that helper (CPU only).

The helper in `q4_q8_int8_amd/csrc/mmq_device.h` sets M0 and declares it clobbered instead of
saving and restoring it. The compiler reserves M0 and does not promise to honour a clobber
of it. So the helper is only correct while the compiler itself neither reads nor writes M0
in the kernels that call it. This test compiles those sources to gfx950 assembly with the
library's own flags and checks every instruction outside the inline-assembly blocks.
"""
import importlib.util
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

_spec = importlib.util.spec_from_file_location(
    "q4_q8_int8_amd_build", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                         "q4_q8_int8_amd", "build.py"))
build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(build)

USERS = ["mmq_gemm.hip", "mmq_gemv.hip"]   # the sources that call dma16
M0 = re.compile(r"\bm0\b")


def assembly(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    flags = [f for f in build.FLAGS if f != "-fPIC"]
    cmd = [build.HIPCC, *flags, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def compiler_m0_uses(path: str) -> list[str]:
    uses, in_asm = [], False
    for line in open(path):
        if "ASMSTART" in line:
            in_asm = True
            continue
        if "ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0].strip()
        if not in_asm and code and not code.startswith(".") and M0.search(code):
            uses.append(code)
    return uses


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not found")
def test_compiler_never_uses_m0():
    tmp = tempfile.mkdtemp(prefix="m0_check_")
    try:
        with ThreadPoolExecutor(len(USERS)) as ex:
            paths = list(ex.map(lambda s: assembly(s, tmp), USERS))
        for src, path in zip(USERS, paths):
            text = open(path).read()
            assert "buffer_load_dwordx4" in text and "lds" in text, f"{src}: no LDS loads found"
            uses = compiler_m0_uses(path)
            assert not uses, f"{src}: the compiler uses M0 outside the helper: {uses[:5]}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_checker_sees_a_compiler_use():
    """The scan itself: an M0 write outside an asm block is reported, one inside is not."""
    tmp = tempfile.mkdtemp(prefix="m0_check_")
    try:
        p = os.path.join(tmp, "x.s")
        with open(p, "w") as f:
            f.write(";;#ASMSTART\n\ts_mov_b32 m0, s2\n;;#ASMEND\n\ts_mov_b32 m0, -1\n"
                    "\tv_mov_b32 v1, v2 ; m0 in a comment\n")
        assert compiler_m0_uses(p) == ["s_mov_b32 m0, -1"]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
