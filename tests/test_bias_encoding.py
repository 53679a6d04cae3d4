"""The integer-to-float step of the GEMM's rescale, checked on the CPU.

The integer MFMA accumulates each block's dot product S onto the constant 0x4B400000, the
bits of 1.5 * 2^23. Read as a float, 0x4B400000 + S is then exactly 12582912 + S, and one
fused multiply-add with the pair (da, nda = -12582912 * da) the prepass stores yields
S * da rounded once: fma((12582912 + S), da, nda) computes (12582912 + S) * da - 12582912 * da
= S * da exactly before its single rounding.

Checked here:
- every |S| a q4_K x q8_1 block can produce (32 * 127 * 15 = 60960) lies in the range where
  the encoding holds;
- for every S in [-2^22, 2^22) the bits 0x4B400000 + S read as float32 equal 12582912 + S;
- nda is exact for every finite binary16 da.
"""
import numpy as np

BIAS_BITS = 0x4B400000
BIAS = 12582912.0


def test_block_dot_bound_inside_the_encoding():
    smax = 32 * 127 * 15
    assert smax == 60960 and smax < 2 ** 22
    assert float(np.uint32(BIAS_BITS).view(np.float32)) == BIAS == 1.5 * 2 ** 23


def test_every_offset_integer_reads_back_exactly():
    s = np.arange(-(1 << 22), 1 << 22, dtype=np.int64)
    f = (BIAS_BITS + s).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.array_equal(f, BIAS + s.astype(np.float64))
    # and just outside, the encoding breaks (a plausible wrong bias would not be caught
    # by the range above alone)
    assert float(np.uint32(BIAS_BITS - (1 << 22) - 1).view(np.float32)) != BIAS - (1 << 22) - 1


def test_nda_exact_for_every_f16():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float64)
    nda = -BIAS * h
    assert np.array_equal(nda.astype(np.float32).astype(np.float64), nda)


def test_fused_rescale_is_one_rounding_of_s_da():
    """The exact value fma sees, (12582912 + S) * da + nda, equals S * da for every S of a
    block and a spread of f16 scales (checked exactly in float64, where all three are
    representable)."""
    rng = np.random.default_rng(3)
    s = np.arange(-60960, 60961, dtype=np.float64)
    bits = np.concatenate([rng.integers(1, 0x7C00, 64), [1, 0x03FF, 0x0400, 0x3C00, 0x7BFF]])
    for b in bits.astype(np.uint16):
        da = float(np.uint16(b).view(np.float16))
        exact = (BIAS + s) * da + (-BIAS * da)
        assert np.array_equal(exact, s * da)
