"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a hand-derived fixture (tests/golden/), a closed
form, brute force on tiny inputs, or an exact integer special case. The mutation tests
in test_oracle_mutations.py check that plausible mistakes planted in the oracle make at
least one of these pins fail.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _x_from_bits(hexes):
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


# ----------------------------------------------------------------------------- float16
def _f16_exact_value(bits: int) -> Fraction | float:
    """IEEE binary16 definition: sign, 5-bit biased exponent, 10-bit fraction."""
    s = -1 if bits >> 15 else 1
    e = (bits >> 10) & 31
    f = bits & 1023
    if e == 31:
        return float("nan") if f else s * float("inf")
    if e == 0:
        return s * Fraction(f, 1024) * Fraction(1, 2 ** 14)
    return s * (1 + Fraction(f, 1024)) * (Fraction(2) ** (e - 15))


def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_decode(bits)
    for b in range(65536):
        want = _f16_exact_value(b)
        if isinstance(want, float) and math.isnan(want):
            assert math.isnan(got[b])
        elif isinstance(want, float):
            assert got[b] == want
        else:
            assert Fraction(float(got[b])) == want, hex(b)


# (exact value, bit pattern) of every finite non-negative f16, in increasing order
_F16_POS = [(_f16_exact_value(b), b) for b in range(0x7C00)]


def _f16_rne_bruteforce(x: float) -> float:
    """Nearest f16 by exhaustive search over all finite values, ties to the even bit pattern."""
    fx = Fraction(x)
    s = -1 if fx < 0 else 1
    ax = abs(fx)
    # 65520 is halfway between 65504 (largest finite) and 65536; ties-to-even overflows to inf
    if ax >= 65520:
        return s * float("inf")
    lo_val, lo_bits = max((p for p in _F16_POS if p[0] <= ax), key=lambda p: p[0])
    if lo_val == ax:
        return float(s * lo_val)
    hi_val, hi_bits = min((p for p in _F16_POS if p[0] > ax), key=lambda p: p[0])
    if ax - lo_val < hi_val - ax:
        return float(s * lo_val)
    if hi_val - ax < ax - lo_val:
        return float(s * hi_val)
    return float(s * (lo_val if lo_bits % 2 == 0 else hi_val))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (65520.0, 0x7C00), (65519.99, 0x7BFF),
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (1.5 * 2.0 ** -25, 0x0001),
    (1.0 + 2.0 ** -11, 0x3C00), (1.0 + 3 * 2.0 ** -11, 0x3C02), (0.5, 0x3800),
    (2.0 ** -14, 0x0400), (0.0, 0x0000), (-0.0, 0x8000),
])
def test_f16_encode_closed_forms(x, bits):
    assert int(oracle.f16_encode(np.float32(x))) == bits


def test_f16_encode_random_vs_bruteforce():
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.uniform(-3, 3, 60), rng.uniform(-1e-6, 1e-6, 30),
                         np.exp(rng.uniform(-20, 11, 60)) * rng.choice([-1, 1], 60)]).astype(np.float32)
    got = oracle.f16_decode(oracle.f16_encode(xs))
    for x, g in zip(xs, got):
        assert g == _f16_rne_bruteforce(float(x)), float(x)


# ----------------------------------------------------------------------------- q8_1
def _golden_q8(golden_dir):
    with open(os.path.join(golden_dir, "q8_1_worked_blocks.json")) as f:
        return json.load(f)["blocks"]


def test_q8_1_hand_derived_blocks(golden_dir):
    blocks = _golden_q8(golden_dir)
    x = np.stack([_x_from_bits(b["x_f32_bits"]) for b in blocks])          # [nblk, 32]
    q = oracle.quantize_q8_1(x)                                             # one row per block
    for i, b in enumerate(blocks):
        assert q.qs[i].tolist() == b["q"], b["name"]
        assert int(q.sa[i, 0]) == b["sa"], b["name"]
        assert int(q.da_bits[i, 0]) == int(b["da_bits"], 16), b["name"]
    # the same blocks laid along K in one row give the same per-block results
    row = oracle.quantize_q8_1(x.reshape(1, -1))
    assert np.array_equal(row.qs.reshape(len(blocks), 32), q.qs)
    assert np.array_equal(row.sa.reshape(-1), q.sa.reshape(-1))


def test_q8_1_invariants_random():
    x = synth.activations("normal_outliers", 64, 1024, 11)
    x[3, :32] = 0.0                                   # an all-zero block
    q = oracle.quantize_q8_1(x)
    xb = x.reshape(64, 32, 32).astype(np.float64)
    qs = q.qs.reshape(64, 32, 32).astype(np.int64)
    amax = np.abs(xb).max(axis=2)
    nz = amax > 0
    # every nonzero block reaches the full range, |q| <= 127 everywhere
    assert np.all(np.abs(qs).max(axis=2)[nz] == 127)
    assert np.all(np.abs(qs) <= 127)
    assert np.all(qs[~nz] == 0)
    # sa is the integer block sum
    assert np.array_equal(q.sa, qs.sum(axis=2))
    assert np.all(np.abs(q.sa) <= 4064)
    # reconstruction error: |q*d - x| <= d/2 up to f32 rounding of the scale (d = amax/127)
    d = amax / 127.0
    err = np.abs(qs * d[..., None] - xb)
    assert np.all(err <= d[..., None] * (0.5 + 1e-5) + 1e-30)
    # sign is preserved and the map is monotone inside a block
    assert np.all((np.sign(qs) == np.sign(xb)) | (qs == 0))
    order = np.argsort(xb, axis=2, kind="stable")
    qsorted = np.take_along_axis(qs, order, axis=2)
    assert np.all(np.diff(qsorted, axis=2) >= 0)
    # the stored scale is amax/127 rounded to f16 (exact rational check on a sample)
    for i, b in [(0, 0), (5, 7), (63, 31), (17, 12)]:
        d32 = Fraction(float(np.float32(amax[i, b]) / np.float32(127.0)))
        want = _f16_rne_bruteforce(float(d32))
        assert oracle.f16_decode(q.da_bits[i, b]) == want


# ----------------------------------------------------------------------------- q4_K
def _golden_q4k(golden_dir):
    with open(os.path.join(golden_dir, "q4_K_worked_block.json")) as f:
        return json.load(f)


def test_q4_K_hand_packed_block(golden_dir):
    g = _golden_q4k(golden_dir)
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), dtype=np.uint8).reshape(1, 1, 144)
    f = oracle.decode_q4_K(blk)
    assert f.d[0, 0] == g["d"] and f.dmin[0, 0] == g["dmin"]
    assert f.sc[0].tolist() == g["sc"]
    assert f.m[0].tolist() == g["m"]
    want_v = [(b + t) % 16 for b in range(8) for t in range(32)]
    assert f.v[0].tolist() == want_v
    w = oracle.dequantize_q4_K(f)
    for s in g["weights_spot"]:
        assert w[0, s["b"] * 32 + s["t"]] == s["w"], s


def test_q4_K_generator_packs_hand_block(golden_dir):
    """The input generator's packer reproduces the hand-packed bytes (pins synth too)."""
    g = _golden_q4k(golden_dir)
    fields = {
        "d_bits": np.array([[0x3C00]], np.uint16), "dmin_bits": np.array([[0x3800]], np.uint16),
        "sc": np.array([g["sc"]], np.uint8), "m": np.array([g["m"]], np.uint8),
        "v": np.array([[(b + t) % 16 for b in range(8) for t in range(32)]], np.uint8),
    }
    assert synth.q4k_pack(fields).tobytes().hex() == g["bytes_hex"]


def test_q4_K_roundtrip_random_fields():
    f = synth.q4k_random_fields(37, 768, 3)
    dec = oracle.decode_q4_K(synth.q4k_pack(f))
    assert np.array_equal(dec.sc, f["sc"].astype(np.int64))
    assert np.array_equal(dec.m, f["m"].astype(np.int64))
    assert np.array_equal(dec.v, f["v"].astype(np.int64))
    assert np.array_equal(dec.d, f["d_bits"].view(np.float16).astype(np.float64))
    assert np.array_equal(dec.dmin, f["dmin_bits"].view(np.float16).astype(np.float64))


def test_q4_K_dequant_bruteforce_reconstruction():
    """Weights from bytes equal a per-element reconstruction from the generator's fields."""
    f = synth.q4k_random_fields(5, 512, 9)
    w = oracle.dequantize_q4_K(oracle.decode_q4_K(synth.q4k_pack(f)))
    for j in range(5):
        for k in range(512):
            sb, b = k // 256, k // 32
            d = Fraction(float(np.uint16(f["d_bits"][j, sb]).view(np.float16)))
            dmin = Fraction(float(np.uint16(f["dmin_bits"][j, sb]).view(np.float16)))
            want = d * int(f["sc"][j, b]) * int(f["v"][j, k]) - dmin * int(f["m"][j, b])
            assert Fraction(float(w[j, k])) == want


# ----------------------------------------------------------------------------- the product
def _integer_case(M, N, K, seed):
    """d = 1, sc = 1, dmin = 0; integer activations with a +-127 in every block.

    Then amax = 127, d = 1, q = x exactly, da = 1 and every weight is v, so
    C = x @ v^T exactly in integers (|C| < 2^24).
    """
    rng = np.random.default_rng(seed)
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 5] = rng.choice([-127.0, 127.0], (M, K // 32))
    f = {
        "d_bits": np.full((N, K // 256), 0x3C00, np.uint16),
        "dmin_bits": np.zeros((N, K // 256), np.uint16),
        "sc": np.ones((N, K // 32), np.uint8),
        "m": rng.integers(0, 64, (N, K // 32), dtype=np.uint8),
        "v": rng.integers(0, 16, (N, K), dtype=np.uint8),
    }
    return x, f


def test_mmq_integer_special_case_exact():
    x, f = _integer_case(24, 40, 512, 21)
    q = oracle.quantize_q8_1(x)
    assert np.array_equal(q.qs.astype(np.float32), x)
    w = oracle.decode_q4_K(synth.q4k_pack(f))
    want = x.astype(np.int64) @ f["v"].astype(np.int64).T
    assert np.array_equal(oracle.mmq(q, w), want.astype(np.float64))
    ct, T = oracle.mmq_terms(q, w)
    assert np.array_equal(ct, want.astype(np.float64))


def test_block_dots_bruteforce():
    x = synth.activations("normal", 3, 256, 4)
    f = synth.q4k_random_fields(4, 256, 4)
    q = oracle.quantize_q8_1(x)
    w = oracle.decode_q4_K(synth.q4k_pack(f))
    S = oracle.block_dots(q, w, [0, 2], [1, 3, 0])
    for bi in range(8):
        for a, i in enumerate([0, 2]):
            for c, j in enumerate([1, 3, 0]):
                want = 0
                for t in range(32):
                    want += int(q.qs[i, bi * 32 + t]) * int(f["v"][j, bi * 32 + t])
                assert S[bi, a, c] == want


def test_mmq_exact_rational_tiny():
    """Direct and term forms against exact rational arithmetic on a tiny product."""
    x = synth.activations("normal_outliers", 2, 256, 31)
    f = synth.q4k_random_fields(3, 256, 31)
    q = oracle.quantize_q8_1(x)
    w = oracle.decode_q4_K(synth.q4k_pack(f))
    C = oracle.mmq(q, w)
    ct, T = oracle.mmq_terms(q, w)
    for i in range(2):
        for j in range(3):
            exact = Fraction(0)
            tabs = Fraction(0)
            for b in range(8):
                da = Fraction(float(np.uint16(q.da_bits[i, b]).view(np.float16)))
                d = Fraction(float(np.uint16(f["d_bits"][j, 0]).view(np.float16)))
                dmin = Fraction(float(np.uint16(f["dmin_bits"][j, 0]).view(np.float16)))
                for t in range(32):
                    k = b * 32 + t
                    wjk = d * int(f["sc"][j, b]) * int(f["v"][j, k]) - dmin * int(f["m"][j, b])
                    exact += da * int(q.qs[i, k]) * wjk
                S = sum(int(q.qs[i, b * 32 + t]) * int(f["v"][j, b * 32 + t]) for t in range(32))
                tabs += abs(da * d * int(f["sc"][j, b]) * S) + abs(dmin * int(f["m"][j, b]) * da * int(q.sa[i, b]))
            assert abs(Fraction(float(C[i, j])) - exact) <= Fraction(1, 10 ** 14) * tabs
            assert abs(Fraction(float(ct[i, j])) - exact) <= Fraction(1, 10 ** 14) * tabs
            assert abs(Fraction(float(T[i, j])) - tabs) <= Fraction(1, 10 ** 14) * tabs


def test_mmq_direct_equals_term_form():
    """term2 invariant: sum_k a_ik dmv_j,b(k) = sum_b dmv_jb da_ib sa_ib, so both forms agree."""
    W = synth.workload("tiny")
    q = oracle.quantize_q8_1(W["x"])
    w = oracle.decode_q4_K(W["w"])
    C = oracle.mmq(q, w)
    ct, T = oracle.mmq_terms(q, w)
    assert np.all(np.abs(C - ct) <= 1e-12 * T)
    assert np.all(T > 0)


def test_mmq_special_case_zero_scales():
    """sc = 0 removes term1: C = -sum_b dmin*m*da*sa; m = 0 removes term2: C = sum_b d*sc*da*S."""
    x = synth.activations("normal", 5, 512, 8)
    q = oracle.quantize_q8_1(x)
    f = synth.q4k_random_fields(6, 512, 8)
    da = q.da_bits.view(np.float16).astype(np.float64)
    sa = q.sa.astype(np.float64)
    d = np.repeat(f["d_bits"].view(np.float16).astype(np.float64), 8, axis=1)
    dmin = np.repeat(f["dmin_bits"].view(np.float16).astype(np.float64), 8, axis=1)

    f0 = dict(f, sc=np.zeros_like(f["sc"]))
    C0 = oracle.mmq(q, oracle.decode_q4_K(synth.q4k_pack(f0)))
    want0 = -(da * sa) @ (dmin * f["m"]).T
    assert np.allclose(C0, want0, rtol=1e-13, atol=1e-12)

    f1 = dict(f, m=np.zeros_like(f["m"]))
    C1 = oracle.mmq(q, oracle.decode_q4_K(synth.q4k_pack(f1)))
    qs = q.qs.astype(np.int64).reshape(5, 16, 32)
    v = f["v"].astype(np.int64).reshape(6, 16, 32)
    S = np.einsum("ibk,jbk->bij", qs, v)
    want1 = np.einsum("ib,jb,bij->ij", da, d * f["sc"], S)
    assert np.allclose(C1, want1, rtol=1e-13, atol=1e-12)


def test_mmq_gemv_row_selection():
    W = synth.workload("tiny")
    q = oracle.quantize_q8_1(W["x"])
    w = oracle.decode_q4_K(W["w"])
    full = oracle.mmq(q, w)
    assert np.array_equal(oracle.mmq(q, w, rows=[7]), full[7:8])
    ct, T = oracle.mmq_terms(q, w, rows=[3, 100])
    ct_all, T_all = oracle.mmq_terms(q, w)
    assert np.array_equal(ct, ct_all[[3, 100]]) and np.array_equal(T, T_all[[3, 100]])
