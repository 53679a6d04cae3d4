"""Pins of the f16 comparator oracle (oracle/f16_oracle.py) to facts outside itself (CPU only).

- convert_f32_f16: hand-derived IEEE binary16 encodings (ties to even, subnormals,
  overflow) and elementwise shape/order.
- dequantize_q4_K_f16:
  - a hand-packed block with hand-derived f16 results, including a float32 value that
    lands on an f16 tie (tests/golden/q4_K_f16_dequant.json);
  - an exact integer case (d = dmin = 1: every weight is the integer sc*v - m);
  - the one-ulp bound against exact rationals built from the generator's fields.
- gemm_f16: an exact integer case against int64 matrix products, and exact rationals on a
  tiny non-square product.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.conftest import GOLDEN


# ----------------------------------------------------------------------------- conversion
# (f32 value, f16 bits): each derived by hand from the binary16 format (1 sign bit, 5 exponent
# bits with bias 15, 10 significand bits; subnormals are multiples of 2^-24)
_F16_CASES = [
    (1.0, 0x3C00),
    (-2.0, 0xC000),
    (1.0 / 3.0, 0x3555),          # 1/3 = 1.0101...b * 2^-2; 10 bits 0101010101, next bit 0
    (65504.0, 0x7BFF),            # largest finite
    (65519.0, 0x7BFF),            # below the midpoint 65520 of 65504 and 2^16
    (65520.0, 0x7C00),            # the midpoint: ties to even, which is infinity
    (-1e6, 0xFC00),
    (2.0 ** -24, 0x0001),         # smallest subnormal
    (2.0 ** -25, 0x0000),         # half of it: a tie, to the even zero
    (3 * 2.0 ** -26, 0x0001),     # 0.75 * 2^-24 rounds up to 2^-24
    (1.5 * 2.0 ** -24, 0x0002),   # tie between 1 and 2 units: even 2
    (1 + 2.0 ** -11, 0x3C00),     # tie between 1 and 1 + 2^-10: even significand 0
    (1 + 3 * 2.0 ** -11, 0x3C02),  # tie between 1 + 2^-10 and 1 + 2^-9: even 2
    (-0.0, 0x8000),
    (2.0 ** -14, 0x0400),         # smallest normal
]


def test_convert_hand_derived_values():
    x = np.array([v for v, _ in _F16_CASES], dtype=np.float32)
    got = oracle.convert_f32_f16(x)
    for (v, want), g in zip(_F16_CASES, got):
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_convert_keeps_shape_and_order():
    x = np.arange(-7, 8, dtype=np.float32).reshape(3, 5) * np.float32(0.5)
    got = oracle.convert_f32_f16(x)
    assert got.shape == (3, 5)
    # small halves are exact in f16: decoding gives the input back, element by element
    assert np.array_equal(oracle.f16_decode(got), x.astype(np.float64))


# ----------------------------------------------------------------------------- dequantization
def _golden():
    with open(os.path.join(GOLDEN, "q4_K_f16_dequant.json")) as f:
        return json.load(f)


def test_dequant_hand_packed_block():
    g = _golden()
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), dtype=np.uint8).reshape(1, 1, 144)
    w = oracle.decode_q4_K(blk)
    assert float(w.d[0, 0]) == g["d"] and float(w.dmin[0, 0]) == g["dmin"]
    assert (w.sc == g["sc"]).all() and (w.m == g["m"]).all()
    assert (w.v.reshape(8, 32) == np.arange(32) % 16).all()
    bits = oracle.dequantize_q4_K_f16(w)
    assert bits.shape == (1, 256) and bits.dtype == np.uint16
    for s in g["spot"]:
        k = 32 * s["b"] + s["t"]
        assert int(bits[0, k]) == int(s["f16_bits"], 16), s
        if "single_rounding_f16_bits" in s:
            # the reading (two roundings) is the one taken, not the single rounding
            assert int(bits[0, k]) != int(s["single_rounding_f16_bits"], 16)


def test_dequant_integer_case_exact():
    """d = dmin = 1 (f16 0x3C00): every weight is the integer sc*v - m, exact in f16."""
    rng = np.random.default_rng(31)
    N, K = 6, 512
    f = {
        "d_bits": np.full((N, K // 256), 0x3C00, np.uint16),
        "dmin_bits": np.full((N, K // 256), 0x3C00, np.uint16),
        "sc": rng.integers(0, 64, (N, K // 32), dtype=np.uint8),
        "m": rng.integers(0, 64, (N, K // 32), dtype=np.uint8),
        "v": rng.integers(0, 16, (N, K), dtype=np.uint8),
    }
    bits = oracle.dequantize_q4_K_f16(oracle.decode_q4_K(synth.q4k_pack(f)))
    want = (np.repeat(f["sc"].astype(np.int64), 32, axis=1) * f["v"].astype(np.int64)
            - np.repeat(f["m"].astype(np.int64), 32, axis=1))
    assert np.array_equal(oracle.f16_decode(bits), want.astype(np.float64))


def _f16_neighbours(x: Fraction):
    """The two adjacent f16 values bracketing x (equal when x is an f16 value), as Fractions."""
    a = abs(x)
    e = -14
    while a >= Fraction(2) ** (e + 1) and e < 15:
        e += 1
    ulp = Fraction(2) ** (e - 10)          # spacing of f16 values around |x|
    lo = (a // ulp) * ulp
    hi = lo if lo == a else lo + ulp
    return (lo, hi, ulp) if x >= 0 else (-hi, -lo, ulp)


def test_dequant_within_one_ulp_of_the_exact_value():
    """Random fields: the f16 value is a neighbour of the exact d*sc*v - dmin*m, and the
    nearest one unless the exact value lies within one float32 spacing of an f16 midpoint."""
    f = synth.q4k_random_fields(4, 512, 77)
    bits = oracle.dequantize_q4_K_f16(oracle.decode_q4_K(synth.q4k_pack(f)))
    got = oracle.f16_decode(bits)
    for j in range(4):
        for k in range(512):
            sb, b = k // 256, k // 32
            d = Fraction(float(np.uint16(f["d_bits"][j, sb]).view(np.float16)))
            dmin = Fraction(float(np.uint16(f["dmin_bits"][j, sb]).view(np.float16)))
            x = d * int(f["sc"][j, b]) * int(f["v"][j, k]) - dmin * int(f["m"][j, b])
            lo, hi, ulp = _f16_neighbours(x)
            g = Fraction(float(got[j, k]))
            assert g in (lo, hi), (j, k)
            mid = (lo + hi) / 2
            if abs(x - mid) > ulp * Fraction(2) ** -12 and lo != hi:
                assert g == (lo if abs(x - lo) < abs(x - hi) else hi), (j, k)


# ----------------------------------------------------------------------------- the GEMM
def test_gemm_integer_case_exact():
    """Small integers are exact f16 values: C and T equal int64 matrix products."""
    rng = np.random.default_rng(5)
    a = rng.integers(-40, 41, (7, 96))
    w = rng.integers(-30, 31, (5, 96))
    C, T = oracle.gemm_f16(oracle.convert_f32_f16(a.astype(np.float32)),
                           oracle.convert_f32_f16(w.astype(np.float32)))
    assert C.shape == (7, 5)
    assert np.array_equal(C, (a @ w.T).astype(np.float64))
    assert np.array_equal(T, (np.abs(a) @ np.abs(w).T).astype(np.float64))


def test_gemm_exact_rationals_tiny():
    rng = np.random.default_rng(6)
    a_bits = oracle.convert_f32_f16(rng.standard_normal((3, 11)).astype(np.float32))
    w_bits = oracle.convert_f32_f16(rng.standard_normal((4, 11)).astype(np.float32) * 0.02)
    C, T = oracle.gemm_f16(a_bits, w_bits)
    a = [[Fraction(float(v)) for v in row] for row in oracle.f16_decode(a_bits)]
    w = [[Fraction(float(v)) for v in row] for row in oracle.f16_decode(w_bits)]
    for i in range(3):
        for j in range(4):
            exact = sum(a[i][k] * w[j][k] for k in range(11))
            tabs = sum(abs(a[i][k] * w[j][k]) for k in range(11))
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(1, 2 ** 50) * tabs
            assert abs(Fraction(T[i, j]) - tabs) <= Fraction(1, 2 ** 50) * tabs


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 1)])
def test_gemm_degenerate_shapes(shape):
    M, N, K = shape
    a = np.full((M, K), 2.0, np.float32)
    w = np.full((N, K), -0.5, np.float32)
    C, T = oracle.gemm_f16(oracle.convert_f32_f16(a), oracle.convert_f32_f16(w))
    assert np.array_equal(C, np.full((M, N), -1.0 * K))
    assert np.array_equal(T, np.full((M, N), 1.0 * K))
