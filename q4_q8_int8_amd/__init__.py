"""q4_K x q8_1 quantized matrix multiply (MMQ) on MI355X (gfx950).

A thin ctypes binding over libmmq.so, whose C ABI is declared in include/mmq.h (the integer
product) and include/mmq_f16.h (the f16 comparator path). The functions here have the same
names and arguments as the C entry points and only marshal arguments: each tensor is checked
(a contiguous CUDA tensor on the current device, of the expected dtype and at least the size
the call reads or writes; MMQArgumentError otherwise) and passed as a device pointer, the
stream defaults to torch's current stream, and a nonzero status raises MMQError. Every step of the computation runs in the
library's HIP kernels; there is no fallback path. Importing this package fails loudly when
libmmq.so has not been built (python q4_q8_int8_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmmq.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_PKG), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "mmq.h")
HEADER_PATHS = (HEADER_PATH, os.path.join(INCLUDE_DIR, "mmq_f16.h"))

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python q4_q8_int8_amd/build.py`")
# torch ships its own HIP runtime. Loading torch first makes libmmq.so's libamdhip64
# dependency resolve to that already-loaded runtime, so the process has a single HIP runtime
# and torch's device pointers and streams are valid in the library's calls. (Loaded the other
# way round, the process would hold two runtimes and the second sees no device.)
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

MMQ_OK, MMQ_E_ARG, MMQ_E_SHAPE, MMQ_E_LDS, MMQ_E_DEVICE, MMQ_E_HIP = range(6)
(MMQ_TILE_AUTO, MMQ_TILE_LARGE, MMQ_TILE_SMALL, MMQ_TILE_SKINNY, MMQ_TILE_GEMV,
 MMQ_TILE_MEDIUM, MMQ_TILE_HALF) = range(7)
(MMQ_REASON_NONE, MMQ_REASON_LARGE, MMQ_REASON_SMALL_GRID, MMQ_REASON_LDS_FALLBACK,
 MMQ_REASON_FORCED, MMQ_REASON_NO_FIT, MMQ_REASON_FEW_TOKENS, MMQ_REASON_FUSED,
 MMQ_REASON_DECODE, MMQ_REASON_SPLIT_K) = range(10)
GEMV_MAX_M = 16  # largest M of the decode tile, which the guard chooses up to there
QK8, QK_K, Q4K_BLOCK_BYTES, REP_TILE_ROWS, REP_TILE_BYTES = 32, 256, 144, 32, 4608
Q6K_BLOCK_BYTES, REP6_TILE_BYTES = 210, 10240


class mmq_options(ctypes.Structure):
    _fields_ = [("force_tile", ctypes.c_int32), ("min_workgroups", ctypes.c_int32),
                ("lds_budget", ctypes.c_int64), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_int64), ("splits", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class mmq_kernel_info(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("reason", ctypes.c_int32),
                ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("fallback", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int64), ("lds_budget", ctypes.c_int64),
                ("grid", ctypes.c_int64), ("splits", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class MMQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        detail = _lib.mmq_last_error().decode()
        super().__init__(f"{fn}: {_lib.mmq_status_str(status).decode()}"
                         + (f" ({detail})" if detail else ""))


_i64, _vp, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "mmq_q8_1_bytes": [_i64, _i64, ctypes.POINTER(_sz)],
    "mmq_q4K_bytes": [_i64, _i64, ctypes.POINTER(_sz)],
    "mmq_q4K_repacked_bytes": [_i64, _i64, ctypes.POINTER(_sz)],
    "quantize_q8_1": [_vp, _i64, _i64, _vp, _vp],
    "repack_q4_K": [_vp, _i64, _i64, _vp, _vp],
    "mmq_q4K_q8_1": [_i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "mmq_q4K_q8_1_ex": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.POINTER(mmq_options)],
    "mmq_q4K_f32": [_i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "mmq_workspace_bytes": [_i64, _i64, _i64, ctypes.POINTER(_sz)],
    "mmq_q6K_bytes": [_i64, _i64, ctypes.POINTER(_sz)],
    "mmq_q6K_repacked_bytes": [_i64, _i64, ctypes.POINTER(_sz)],
    "repack_q6_K": [_vp, _i64, _i64, _vp, _vp],
    "mmq_q6K_q8_1": [_i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "mmq_q6K_q8_1_ex": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.POINTER(mmq_options)],
    "mmq_q6K_q8_1_blockdots": [_i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp,
                               ctypes.POINTER(mmq_options)],
    "mmq_q4K_q8_1_static": [_i64, _i64, _i64, _vp, _vp, _vp, _vp, ctypes.POINTER(mmq_options)],
    "mmq_q4K_q8_1_blockdots": [_i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp,
                               ctypes.POINTER(mmq_options)],
    "mmq_plan": [_i64, _i64, _i64, ctypes.POINTER(mmq_options), _i64,
                 ctypes.POINTER(mmq_kernel_info)],
    "mmq_last_kernel": [ctypes.POINTER(mmq_kernel_info)],
    "mmq_f16_bytes": [_i64, _i64, ctypes.POINTER(_sz)],
    "convert_f32_f16": [_vp, _i64, _i64, _vp, _vp],
    "dequantize_q4_K_f16": [_vp, _i64, _i64, _vp, _vp],
    "gemm_f16": [_i64, _i64, _i64, _vp, _vp, _vp, _vp],
    "mmq_status_str": [ctypes.c_int],
    "mmq_last_error": [],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_char_p if _name in ("mmq_status_str", "mmq_last_error") else ctypes.c_int


def exported_symbols() -> list[str]:
    """Function names declared in the library's headers (include/mmq.h, include/mmq_f16.h)."""
    names = []
    for path in HEADER_PATHS:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return names


def _check(fn: str, status: int) -> None:
    if status != MMQ_OK:
        raise MMQError(fn, status)


class MMQArgumentError(ValueError):
    """A tensor handed to a wrapper does not fit the call (raised before any launch)."""


def _dev(t, name: str, nbytes: int, dtype=None) -> int:
    """Device pointer of tensor t after checking that the call may use it: a contiguous CUDA
    tensor on the current device, of `dtype` when given, holding at least `nbytes` bytes.
    The C ABI takes bare pointers and cannot check buffer sizes itself, so an undersized or
    mistyped buffer is refused here rather than read or written out of bounds."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise MMQArgumentError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise MMQArgumentError(f"{name}: dtype must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MMQArgumentError(f"{name}: must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise MMQArgumentError(f"{name}: holds {have} bytes, the call needs {nbytes}")
    if not t.is_cuda:
        raise MMQArgumentError(f"{name}: must be a CUDA tensor (got device {t.device})")
    if t.device.index != torch.cuda.current_device():
        raise MMQArgumentError(f"{name}: on {t.device}, but the current device is "
                               f"cuda:{torch.cuda.current_device()}")
    return t.data_ptr()


def _f32():
    import torch
    return torch.float32


def _i32():
    import torch
    return torch.int32


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _opts(force_tile: int = MMQ_TILE_AUTO, lds_budget: int = 0, min_workgroups: int = 0,
          workspace: int | None = None, workspace_bytes: int = 0, splits: int = 0):
    if (force_tile == MMQ_TILE_AUTO and lds_budget == 0 and min_workgroups == 0
            and workspace_bytes == 0 and splits == 0):
        return None
    return ctypes.byref(mmq_options(force_tile, min_workgroups, lds_budget, workspace,
                                    workspace_bytes, splits, 0))


def _workspace(workspace):
    """(pointer, bytes) of an optional split-K workspace tensor (a contiguous CUDA tensor)."""
    if workspace is None:
        return None, 0
    nbytes = workspace.numel() * workspace.element_size()
    return _dev(workspace, "workspace", 0), nbytes


# ---------------------------------------------------------------- sizes
def mmq_q8_1_bytes(M: int, K: int) -> int:
    n = _sz()
    _check("mmq_q8_1_bytes", _lib.mmq_q8_1_bytes(M, K, ctypes.byref(n)))
    return n.value


def mmq_q4K_bytes(N: int, K: int) -> int:
    n = _sz()
    _check("mmq_q4K_bytes", _lib.mmq_q4K_bytes(N, K, ctypes.byref(n)))
    return n.value


def mmq_q4K_repacked_bytes(N: int, K: int) -> int:
    n = _sz()
    _check("mmq_q4K_repacked_bytes", _lib.mmq_q4K_repacked_bytes(N, K, ctypes.byref(n)))
    return n.value


# ---------------------------------------------------------------- the hot path
def _gemm_ptrs(M: int, N: int, K: int, q8, w_rep, C):
    return (_dev(q8, "q8", mmq_q8_1_bytes(M, K)),
            _dev(w_rep, "w_rep", mmq_q4K_repacked_bytes(N, K)),
            _dev(C, "C", 4 * M * N, _f32()))


def quantize_q8_1(x, M: int, K: int, q8, stream=None) -> None:
    """x: f32 [M, K] device tensor; q8: device buffer of mmq_q8_1_bytes(M, K) bytes."""
    xp = _dev(x, "x", 4 * M * K, _f32())
    qp = _dev(q8, "q8", mmq_q8_1_bytes(M, K))
    _check("quantize_q8_1", _lib.quantize_q8_1(xp, M, K, qp, _stream(stream)))


def repack_q4_K(w_q4K, N: int, K: int, w_rep, stream=None) -> None:
    """w_q4K: q4_K blocks (mmq_q4K_bytes); w_rep: mmq_q4K_repacked_bytes(N, K) bytes."""
    wp = _dev(w_q4K, "w_q4K", mmq_q4K_bytes(N, K))
    rp = _dev(w_rep, "w_rep", mmq_q4K_repacked_bytes(N, K))
    _check("repack_q4_K", _lib.repack_q4_K(wp, N, K, rp, _stream(stream)))


def mmq_q4K_q8_1(M: int, N: int, K: int, q8, w_rep, C, stream=None) -> None:
    """C[M, N] (f32 device tensor) = q8 (M x K) times repacked q4_K weights (N x K)^T."""
    qp, rp, cp = _gemm_ptrs(M, N, K, q8, w_rep, C)
    _check("mmq_q4K_q8_1", _lib.mmq_q4K_q8_1(M, N, K, qp, rp, cp, _stream(stream)))


def mmq_q4K_q8_1_ex(M: int, N: int, K: int, q8, w_rep, C, stream=None,
                    force_tile: int = MMQ_TILE_AUTO, lds_budget: int = 0,
                    min_workgroups: int = 0, workspace=None, splits: int = 0) -> None:
    """As mmq_q4K_q8_1 with options; `workspace` (any contiguous CUDA tensor, its whole byte
    size usable) lets the guard split K over workgroups, `splits` forces a split count."""
    qp, rp, cp = _gemm_ptrs(M, N, K, q8, w_rep, C)
    wp, wb = _workspace(workspace)
    _check("mmq_q4K_q8_1_ex",
           _lib.mmq_q4K_q8_1_ex(M, N, K, qp, rp, cp, _stream(stream),
                                _opts(force_tile, lds_budget, min_workgroups, wp, wb, splits)))


def mmq_q4K_q8_1_static(M: int, N: int, K: int, q8, w_rep, C, stream=None,
                        force_tile: int = MMQ_TILE_AUTO, lds_budget: int = 0,
                        min_workgroups: int = 0, splits: int = 0) -> None:
    """As mmq_q4K_q8_1_ex, the split-K workspace being the library's own 32 MiB device array
    (for callers that cannot allocate); calls that overlap on one GPU race."""
    qp, rp, cp = _gemm_ptrs(M, N, K, q8, w_rep, C)
    _check("mmq_q4K_q8_1_static",
           _lib.mmq_q4K_q8_1_static(M, N, K, qp, rp, cp, _stream(stream),
                                    _opts(force_tile, lds_budget, min_workgroups, None, 0,
                                          splits)))


def mmq_workspace_bytes(M: int, N: int, K: int) -> int:
    """Split-K workspace the guard would use for M x N x K given an unlimited one (0: none)."""
    n = _sz()
    _check("mmq_workspace_bytes", _lib.mmq_workspace_bytes(M, N, K, ctypes.byref(n)))
    return n.value


def mmq_q4K_f32(M: int, N: int, K: int, x, w_rep, C, stream=None) -> None:
    """Few tokens (M <= 128): C[M, N] from f32 activations x [M, K], quantized in the GEMM."""
    xp = _dev(x, "x", 4 * M * K, _f32())
    rp = _dev(w_rep, "w_rep", mmq_q4K_repacked_bytes(N, K))
    cp = _dev(C, "C", 4 * M * N, _f32())
    _check("mmq_q4K_f32", _lib.mmq_q4K_f32(M, N, K, xp, rp, cp, _stream(stream)))


def mmq_q4K_q8_1_blockdots(M: int, N: int, K: int, q8, w_rep, i0: int, i1: int, j0: int,
                           j1: int, S, stream=None, force_tile: int = MMQ_TILE_AUTO,
                           lds_budget: int = 0) -> None:
    """S: int32 device tensor [K/32, i1-i0, j1-j0] of per-block integer dot products."""
    qp = _dev(q8, "q8", mmq_q8_1_bytes(M, K))
    rp = _dev(w_rep, "w_rep", mmq_q4K_repacked_bytes(N, K))
    sp = _dev(S, "S", 4 * (K // QK8) * max(i1 - i0, 0) * max(j1 - j0, 0), _i32())
    _check("mmq_q4K_q8_1_blockdots",
           _lib.mmq_q4K_q8_1_blockdots(M, N, K, qp, rp, i0, i1, j0, j1, sp,
                                       _stream(stream), _opts(force_tile, lds_budget)))


# ---------------------------------------------------------------- the q6_K variant
def mmq_q6K_bytes(N: int, K: int) -> int:
    n = _sz()
    _check("mmq_q6K_bytes", _lib.mmq_q6K_bytes(N, K, ctypes.byref(n)))
    return n.value


def mmq_q6K_repacked_bytes(N: int, K: int) -> int:
    n = _sz()
    _check("mmq_q6K_repacked_bytes", _lib.mmq_q6K_repacked_bytes(N, K, ctypes.byref(n)))
    return n.value


def repack_q6_K(w_q6K, N: int, K: int, w_rep, stream=None) -> None:
    """w_q6K: q6_K blocks (mmq_q6K_bytes); w_rep: mmq_q6K_repacked_bytes(N, K) bytes."""
    wp = _dev(w_q6K, "w_q6K", mmq_q6K_bytes(N, K))
    rp = _dev(w_rep, "w_rep", mmq_q6K_repacked_bytes(N, K))
    _check("repack_q6_K", _lib.repack_q6_K(wp, N, K, rp, _stream(stream)))


def _gemm6_ptrs(M: int, N: int, K: int, q8, w_rep, C):
    return (_dev(q8, "q8", mmq_q8_1_bytes(M, K)),
            _dev(w_rep, "w_rep", mmq_q6K_repacked_bytes(N, K)),
            _dev(C, "C", 4 * M * N, _f32()))


def mmq_q6K_q8_1(M: int, N: int, K: int, q8, w_rep, C, stream=None) -> None:
    """C[M, N] (f32) = q8 (M x K) times repacked q6_K weights (N x K)^T."""
    qp, rp, cp = _gemm6_ptrs(M, N, K, q8, w_rep, C)
    _check("mmq_q6K_q8_1", _lib.mmq_q6K_q8_1(M, N, K, qp, rp, cp, _stream(stream)))


def mmq_q6K_q8_1_ex(M: int, N: int, K: int, q8, w_rep, C, stream=None,
                    force_tile: int = MMQ_TILE_AUTO, lds_budget: int = 0,
                    min_workgroups: int = 0, workspace=None, splits: int = 0) -> None:
    qp, rp, cp = _gemm6_ptrs(M, N, K, q8, w_rep, C)
    wp, wb = _workspace(workspace)
    _check("mmq_q6K_q8_1_ex",
           _lib.mmq_q6K_q8_1_ex(M, N, K, qp, rp, cp, _stream(stream),
                                _opts(force_tile, lds_budget, min_workgroups, wp, wb, splits)))


def mmq_q6K_q8_1_blockdots(M: int, N: int, K: int, q8, w_rep, i0: int, i1: int, j0: int,
                           j1: int, S, stream=None, force_tile: int = MMQ_TILE_AUTO) -> None:
    """S: int32 device tensor [K/16, i1-i0, j1-j0] of per-group integer dot products."""
    qp = _dev(q8, "q8", mmq_q8_1_bytes(M, K))
    rp = _dev(w_rep, "w_rep", mmq_q6K_repacked_bytes(N, K))
    sp = _dev(S, "S", 4 * (K // 16) * max(i1 - i0, 0) * max(j1 - j0, 0), _i32())
    _check("mmq_q6K_q8_1_blockdots",
           _lib.mmq_q6K_q8_1_blockdots(M, N, K, qp, rp, i0, i1, j0, j1, sp, _stream(stream),
                                       _opts(force_tile)))


# ---------------------------------------------------------------- the guard
def mmq_plan(M: int, N: int, K: int, lds_budget: int, force_tile: int = MMQ_TILE_AUTO,
             opt_lds_budget: int = 0, min_workgroups: int = 0, workspace_bytes: int = 0,
             splits: int = 0) -> dict:
    info = mmq_kernel_info()
    _check("mmq_plan", _lib.mmq_plan(M, N, K, _opts(force_tile, opt_lds_budget, min_workgroups,
                                                    None, workspace_bytes, splits),
                                     lds_budget, ctypes.byref(info)))
    return info.as_dict()


# ---------------------------------------------------------------- the f16 comparator path
def mmq_f16_bytes(rows: int, K: int) -> int:
    n = _sz()
    _check("mmq_f16_bytes", _lib.mmq_f16_bytes(rows, K, ctypes.byref(n)))
    return n.value


def convert_f32_f16(x, M: int, K: int, x_f16, stream=None) -> None:
    """x: f32 [M, K] device tensor; x_f16: device buffer of mmq_f16_bytes(M, K) bytes."""
    xp = _dev(x, "x", 4 * M * K, _f32())
    hp = _dev(x_f16, "x_f16", mmq_f16_bytes(M, K))
    _check("convert_f32_f16", _lib.convert_f32_f16(xp, M, K, hp, _stream(stream)))


def dequantize_q4_K_f16(w_q4K, N: int, K: int, w_f16, stream=None) -> None:
    """w_q4K: q4_K blocks (mmq_q4K_bytes); w_f16: mmq_f16_bytes(N, K) bytes."""
    wp = _dev(w_q4K, "w_q4K", mmq_q4K_bytes(N, K))
    hp = _dev(w_f16, "w_f16", mmq_f16_bytes(N, K))
    _check("dequantize_q4_K_f16", _lib.dequantize_q4_K_f16(wp, N, K, hp, _stream(stream)))


def gemm_f16(M: int, N: int, K: int, x_f16, w_f16, C, stream=None) -> None:
    """C[M, N] (f32 device tensor) = x_f16 [M, K] times w_f16 [N, K]^T, f32 accumulation."""
    xp = _dev(x_f16, "x_f16", mmq_f16_bytes(M, K))
    wp = _dev(w_f16, "w_f16", mmq_f16_bytes(N, K))
    cp = _dev(C, "C", 4 * M * N, _f32())
    _check("gemm_f16", _lib.gemm_f16(M, N, K, xp, wp, cp, _stream(stream)))


def mmq_last_kernel() -> dict:
    info = mmq_kernel_info()
    _check("mmq_last_kernel", _lib.mmq_last_kernel(ctypes.byref(info)))
    return info.as_dict()


def mmq_status_str(status: int) -> str:
    return _lib.mmq_status_str(status).decode()


def mmq_last_error() -> str:
    return _lib.mmq_last_error().decode()


def raw_call(name: str, *args) -> int:
    """Call a C entry point by name with raw ctypes-compatible arguments; returns the status."""
    return getattr(_lib, name)(*args)
