"""The host ABI tests again, with api.cpp built under AddressSanitizer and UBSan (CPU only).

api.cpp holds the library's host logic: argument validation, the overflow-checked size
arithmetic, the tile guard and its cost model, the per-thread error text. This builds a
copy of libmmq.so whose api.cpp object is instrumented (host code only: each -fsanitize=
flag is passed through -Xarch_host; the kernels are built as usual), puts it in a temporary
copy of the package, and runs tests/test_abi_host.py against it in a child process with the
ASan runtime preloaded. Any sanitizer report aborts the child and fails this test.
"""
import importlib.util
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location(
    "q4_q8_int8_amd_build_san", os.path.join(ROOT, "q4_q8_int8_amd", "build.py"))
build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(build)

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
CLANG = os.path.join(os.path.dirname(os.path.realpath(build.HIPCC)), "..", "llvm", "bin",
                     "clang++")

RUNNER = """
import sys
sys.path.insert(0, sys.argv[1])
import q4_q8_int8_amd as m
assert m.LIB_PATH.startswith(sys.argv[1]), m.LIB_PATH
import ctypes
assert hasattr(ctypes.CDLL(None), "__asan_init"), "the ASan runtime is not loaded"
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", sys.argv[2]]))
"""


def _asan_runtime() -> str:
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not found")
def test_host_abi_under_asan_and_ubsan():
    runtime = _asan_runtime()
    if not runtime:
        pytest.skip("no ASan runtime next to the ROCm clang")
    tmp = tempfile.mkdtemp(prefix="mmq_san_")
    try:
        pkg = os.path.join(tmp, "pkg", "q4_q8_int8_amd")
        os.makedirs(pkg)

        def compile_one(src):
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            extra = SAN if src == "api.cpp" else []
            r = subprocess.run([build.HIPCC, *build.FLAGS, *extra, *lang, "-c",
                                os.path.join(build.CSRC, src), "-o", obj],
                               capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            return obj

        with ThreadPoolExecutor(min(8, len(build.SOURCES))) as ex:
            objs = list(ex.map(compile_one, build.SOURCES))
        lib = os.path.join(pkg, "libmmq.so")
        r = subprocess.run([build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                            "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                            "-fsanitize=undefined", "-shared-libasan", *objs, "-o", lib],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
        assert "__asan_report" in nm and "__ubsan_handle" in nm, "api.cpp is not instrumented"
        shutil.copy(os.path.join(ROOT, "q4_q8_int8_amd", "__init__.py"), pkg)
        shutil.copytree(os.path.join(ROOT, "include"), os.path.join(tmp, "pkg", "include"))
        runner = os.path.join(tmp, "run.py")
        with open(runner, "w") as f:
            f.write(RUNNER)
        env = dict(os.environ, LD_PRELOAD=runtime,
                   ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        r = subprocess.run([sys.executable, runner, os.path.join(tmp, "pkg"),
                            os.path.join(ROOT, "tests", "test_abi_host.py")],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
        out = r.stdout + r.stderr
        assert r.returncode == 0, out[-4000:]
        assert "passed" in out and "ERROR: AddressSanitizer" not in out \
            and "runtime error" not in out, out[-4000:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
