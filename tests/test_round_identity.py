"""The rounding step of the GPU quantize kernel for whole super-blocks, checked on the CPU.

That kernel rounds p = x * id half away from zero without a roundf call: it adds
copysign(0.5 - 2^-25, p) in float32 (round to nearest even) and truncates toward zero (the
truncating float-to-int conversion). This file checks that identity against the definition
of half-away rounding, computed exactly in float64:
- every float32 in [2^-4, 4), both signs: around 0.5 the sum crosses into the next binade
  and the addition rounds;
- every float32 within 64 ulps of each half-integer up to 2^24;
- random bit patterns over the whole float32 range.
With MMQ_EXHAUSTIVE=1 it checks all 2^32 bit patterns (a few minutes).
The q8_1 bytes the kernel produces are compared with the oracle by the GPU parity tests.
"""
import os

import numpy as np
import pytest

C = np.float32(0.5) - np.float32(2.0 ** -25)


def kernel_round(p: np.ndarray) -> np.ndarray:
    s = (p + np.copysign(C, p)).astype(np.float32)   # one float32 addition, RNE
    return np.trunc(s).astype(np.float64)


def half_away(p: np.ndarray) -> np.ndarray:
    a = np.abs(p.astype(np.float64))
    return np.copysign(np.floor(a + 0.5), p.astype(np.float64))   # exact in float64


def check(p: np.ndarray):
    p = p[np.isfinite(p)]
    bad = kernel_round(p) != half_away(p)
    assert not bad.any(), f"{int(bad.sum())} mismatches, e.g. {p[bad][:4]}"


def bits_range(lo: float, hi: float) -> np.ndarray:
    a = np.array([lo, hi], np.float32).view(np.uint32)
    return np.arange(a[0], a[1], dtype=np.uint32).view(np.float32)


def test_constant():
    assert float(C) == 0.5 - 2.0 ** -25 and C < 0.5


def test_small_magnitudes_dense():
    p = bits_range(2.0 ** -4, 4.0)               # 6 binades, 5.0e7 values
    for part in np.array_split(p, 16):
        check(part)
        check(-part)


def test_near_half_integers():
    k = np.arange(0, 1 << 24, 997, dtype=np.float64)
    for off in range(-64, 65):
        h = (k + 0.5).astype(np.float32)
        u = h.view(np.int32).astype(np.int64) + off
        p = u.astype(np.int32).view(np.float32)
        check(p)
        check(-p)


def test_random_bit_patterns():
    rng = np.random.default_rng(11)
    check(rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
          .view(np.float32))


@pytest.mark.skipif(os.environ.get("MMQ_EXHAUSTIVE") != "1", reason="set MMQ_EXHAUSTIVE=1")
def test_every_float32():
    for hi in range(256):
        u = (np.arange(1 << 24, dtype=np.uint64) + (hi << 24)).astype(np.uint32)
        check(u.view(np.float32))
