"""Helpers for the GPU tests: device buffers, calls through the C ABI, oracle caching."""
import functools
import json
import os
import sys

import numpy as np
import torch

import oracle
import synth
import q4_q8_int8_amd as mmq

SAMPLE_SEED = 77


def say(*args):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def gpu_quantize(x: np.ndarray) -> torch.Tensor:
    M, K = x.shape
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")  # padding = 0
    mmq.quantize_q8_1(to_dev(x), M, K, q8)
    torch.cuda.synchronize()
    return q8


def gpu_repack(w: np.ndarray, N: int, K: int) -> torch.Tensor:
    assert w.shape == (N, K // 256, 144)
    rep = torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    mmq.repack_q4_K(to_dev(w), N, K, rep)
    torch.cuda.synchronize()
    return rep


def gpu_mmq(M, N, K, q8, rep, force_tile=0, lds_budget=0) -> np.ndarray:
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_q8_1_ex(M, N, K, q8, rep, C, force_tile=force_tile, lds_budget=lds_budget)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def gpu_blockdots(M, N, K, q8, rep, i0, i1, j0, j1, force_tile=0) -> np.ndarray:
    S = torch.full((K // 32, i1 - i0, j1 - j0), -(2 ** 31), dtype=torch.int32, device="cuda")
    mmq.mmq_q4K_q8_1_blockdots(M, N, K, q8, rep, i0, i1, j0, j1, S, force_tile=force_tile)
    torch.cuda.synchronize()
    return S.cpu().numpy()


@functools.lru_cache(maxsize=4)
def workload(name: str):
    return synth.workload(name, need_fields=True)


@functools.lru_cache(maxsize=4)
def oracle_q8(name: str):
    return oracle.quantize_q8_1(workload(name)["x"])


@functools.lru_cache(maxsize=4)
def oracle_w(name: str):
    return oracle.decode_q4_K(workload(name)["w"])


def sample_rows(M: int, n_random: int = 8) -> np.ndarray:
    """Tile-boundary rows plus seeded random rows."""
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, M // 2, M - 129, M - 128, M - 33, M - 1}
    rng = np.random.default_rng(SAMPLE_SEED + M)
    rand = set(rng.integers(0, M, n_random).tolist())
    return np.array(sorted(r for r in fixed | rand if 0 <= r < M))


def assert_within_tolerance(C_gpu: np.ndarray, C_ref: np.ndarray, T: np.ndarray, tol=1e-5):
    """|C_gpu - C_ref| <= tol * T elementwise (T = sum of |terms|); returns the max ratio."""
    assert C_gpu.shape == C_ref.shape == T.shape
    assert np.all(np.isfinite(C_gpu)), "non-finite output"
    err = np.abs(C_gpu.astype(np.float64) - C_ref)
    bad = err > tol * T
    if np.any(bad):
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{bad.sum()} elements outside {tol}*T, first {idx}: "
                             f"gpu={C_gpu[bad][:5]}, ref={C_ref[bad][:5]}, T={T[bad][:5]}")
    pos = T > 0
    r = float((err[pos] / T[pos]).max()) if np.any(pos) else 0.0
    log = os.environ.get("PARITY_LOG")
    if log:   # the measured ratio of each case, for the record of the run
        with open(log, "a") as f:
            f.write(json.dumps({"case": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0],
                                "shape": list(C_gpu.shape), "max_err_over_T": r,
                                "tol": tol}) + "\n")
    return r
