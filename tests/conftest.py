import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (seconds of CPU oracle work)")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def _ensure_built():
    """Build libmmq.so in-tree when it is missing (hipcc cross-compiles without a GPU)."""
    lib = os.path.join(ROOT, "q4_q8_int8_amd", "libmmq.so")
    if not os.path.exists(lib):
        # by path: importing the package needs the library it builds
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "q4_q8_int8_amd_build", os.path.join(ROOT, "q4_q8_int8_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


_ensure_built()
