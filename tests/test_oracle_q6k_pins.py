"""Pins of the q6_K oracle against things other than itself, and planted mistakes (CPU only).

- a hand-packed super-block (tests/golden/q6_K_worked_block.json) whose bytes, fields and
  spot weights are derived by hand in the file;
- the generator's packer and the oracle's decoder are inverse on random fields;
- dequantized weights equal exact rationals built from the generator's fields;
- the integer case d = 1, sc = 1 with integer activations: C = x (u - 32)^T exactly;
- brute-force group dot products;
- the per-group form equals the direct product, and the pages' fold form (unsigned values
  plus a rank-1 correction of the offset) equals both;
- zero scales remove their groups.
Each planted mistake below must make at least one of these fail.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.q6k_oracle as qo
import synth
from tests.conftest import GOLDEN


def _golden():
    with open(os.path.join(GOLDEN, "q6_K_worked_block.json")) as f:
        return json.load(f)


def test_q6_K_hand_packed_block():
    g = _golden()
    # the bytes follow from the derivation in the file
    by_hand = bytes([0x11 * ((i % 32) & 15) for i in range(128)]
                    + [0x88 if (i % 32) < 16 else 0xDD for i in range(64)]
                    + [(k - 8) & 0xFF for k in range(16)] + [0x00, 0x38])
    assert by_hand.hex() == g["bytes_hex"]
    blk = np.frombuffer(bytes.fromhex(g["bytes_hex"]), dtype=np.uint8).reshape(1, 1, 210)
    w = oracle.decode_q6_K(blk)
    assert w.d[0, 0] == 0.5
    assert w.sc[0].tolist() == [k - 8 for k in range(16)]
    assert w.u[0].tolist() == [v % 64 for v in range(256)]
    deq = oracle.dequantize_q6_K(w)
    for s in g["weights_spot"]:
        assert deq[0, s["v"]] == s["w"], s


def test_q6_K_generator_packs_hand_block():
    g = _golden()
    f = {"d_bits": np.array([[0x3800]], np.uint16),
         "sc": np.array([[k - 8 for k in range(16)]], np.int8),
         "u": np.array([[v % 64 for v in range(256)]], np.uint8)}
    assert synth.q6k_pack(f).tobytes().hex() == g["bytes_hex"]


@pytest.mark.parametrize("N,K", [(3, 256), (5, 768), (1, 1024)])
def test_q6_K_roundtrip_random_fields(N, K):
    f = synth.q6k_random_fields(N, K, N * 13 + K)
    w = oracle.decode_q6_K(synth.q6k_pack(f))
    assert np.array_equal(w.u, f["u"].astype(np.int64))
    assert np.array_equal(w.sc, f["sc"].astype(np.int64))
    assert np.array_equal(w.d, f["d_bits"].view(np.float16).astype(np.float64))


def test_q6_K_dequant_bruteforce_reconstruction():
    N, K = 3, 512
    f = synth.q6k_random_fields(N, K, 77)
    deq = oracle.dequantize_q6_K(oracle.decode_q6_K(synth.q6k_pack(f)))
    for j in range(N):
        for k in range(0, K, 7):
            d = Fraction(float(np.uint16(f["d_bits"][j, k // 256]).view(np.float16)))
            want = d * int(f["sc"][j, k // 16]) * (int(f["u"][j, k]) - 32)
            assert Fraction(float(deq[j, k])) == want, (j, k)


def test_mmq_q6K_integer_special_case_exact():
    """d = 1, sc = 1, integer activations with a +-127 in every block: da = 1, q = x, and C is
    the integer product x (u - 32)^T, exactly."""
    rng = np.random.default_rng(5)
    M, N, K = 7, 9, 512
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 3] = rng.choice([-127.0, 127.0], (M, K // 32))
    f = {"d_bits": np.full((N, K // 256), 0x3C00, np.uint16),
         "sc": np.ones((N, K // 16), np.int8),
         "u": rng.integers(0, 64, (N, K), dtype=np.uint8)}
    q = oracle.quantize_q8_1(x)
    w = oracle.decode_q6_K(synth.q6k_pack(f))
    want = x.astype(np.int64) @ (f["u"].astype(np.int64) - 32).T
    assert np.array_equal(oracle.mmq_q6K(q, w), want.astype(np.float64))
    C, T = oracle.mmq_q6K_terms(q, w)
    assert np.array_equal(C, want.astype(np.float64))


def test_block_dots_q6K_bruteforce():
    M, N, K = 3, 4, 256
    x = synth.activations("normal", M, K, 8)
    f = synth.q6k_random_fields(N, K, 9)
    q = oracle.quantize_q8_1(x)
    w = oracle.decode_q6_K(synth.q6k_pack(f))
    S = oracle.block_dots_q6K(q, w, range(M), range(N))
    assert S.shape == (K // 16, M, N)
    for gidx in range(K // 16):
        for i in range(M):
            for j in range(N):
                want = sum(int(q.qs[i, k]) * (int(f["u"][j, k]) - 32)
                           for k in range(16 * gidx, 16 * gidx + 16))
                assert S[gidx, i, j] == want


@pytest.mark.parametrize("kind", ["random_fields", "fit"])
def test_mmq_q6K_forms_agree(kind):
    M, N, K = 40, 33, 1024
    x = synth.activations("normal_outliers", M, K, 11)
    wb, _ = synth.q6k_weights(kind, N, K, 12)
    q = oracle.quantize_q8_1(x)
    w = oracle.decode_q6_K(wb)
    C = oracle.mmq_q6K(q, w)
    C_terms, T = oracle.mmq_q6K_terms(q, w)
    C_fold = oracle.mmq_q6K_fold_terms(q, w)
    assert np.all(T > 0)
    assert np.all(np.abs(C - C_terms) <= 1e-12 * T)
    assert np.all(np.abs(C - C_fold) <= 1e-12 * T)


def test_mmq_q6K_zero_scales():
    M, N, K = 5, 6, 512
    x = synth.activations("normal", M, K, 13)
    f = synth.q6k_random_fields(N, K, 14)
    f["sc"][:, ::2] = 0                      # every even group contributes nothing
    q = oracle.quantize_q8_1(x)
    w = oracle.decode_q6_K(synth.q6k_pack(f))
    C = oracle.mmq_q6K(q, w)
    S = oracle.block_dots_q6K(q, w, range(M), range(N)).astype(np.float64)
    da = oracle.f16_decode(q.da_bits)                        # [M, K/32]
    dsv = oracle.q6_K_scales(w)                              # [N, K/16]
    want = sum(np.outer(da[:, g // 2], dsv[:, g]) * S[g] for g in range(1, K // 16, 2))
    _, T = oracle.mmq_q6K_terms(q, w)
    assert np.all(np.abs(C - want) <= 1e-12 * T)


# ----------------------------------------------------------------------------- planted mistakes
PINS = {
    "golden": test_q6_K_hand_packed_block,
    "roundtrip": lambda: test_q6_K_roundtrip_random_fields(5, 768),
    "bruteforce": test_q6_K_dequant_bruteforce_reconstruction,
    "int_case": test_mmq_q6K_integer_special_case_exact,
    "block_dots": test_block_dots_q6K_bruteforce,
    "forms": lambda: test_mmq_q6K_forms_agree("random_fields"),
    "zero_scales": test_mmq_q6K_zero_scales,
}

_ORIG = {"decode": qo.decode_q6_K, "scales": qo.q6_K_scales, "dots": qo.block_dots_q6K}


def _decode_mut(kind):
    def f(blocks):
        w = _ORIG["decode"](blocks)
        u, sc = w.u.copy(), w.sc.copy()
        N, K = u.shape
        u5 = u.reshape(N, K // 256, 2, 4, 32)
        if kind == "hi_nibble_quarters_swapped":   # values 64.. read from the wrong nibble
            u5[:, :, :, [2, 3], :] = u5[:, :, :, [3, 2], :].copy()
        if kind == "high_bits_dropped":
            u = u & 15
            return qo.Q6K(d=w.d, sc=sc, u=u)
        if kind == "scale_per_32":                # one scale per 32 values instead of 16
            sc = np.repeat(sc[:, ::2], 2, axis=1)
        return qo.Q6K(d=w.d, sc=sc, u=u5.reshape(N, K))
    return f


def _dequant_no_offset(w):
    dsv = qo.q6_K_scales(w)
    N, K = w.u.shape
    return (dsv[..., None] * w.u.reshape(N, K // 16, 16)).reshape(N, K)


def _dots_unsigned(q, w, rows, cols):
    return _ORIG["dots"](q, qo.Q6K(d=w.d, sc=w.sc, u=w.u + 32), rows, cols)


MUTATIONS = {
    "hi_nibble_quarters_swapped": ("decode_q6_K", _decode_mut("hi_nibble_quarters_swapped")),
    "high_bits_dropped": ("decode_q6_K", _decode_mut("high_bits_dropped")),
    "scale_per_32": ("decode_q6_K", _decode_mut("scale_per_32")),
    "offset_dropped": ("dequantize_q6_K", _dequant_no_offset),
    "dots_without_offset": ("block_dots_q6K", _dots_unsigned),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_q6K_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(qo, attr, bad)
    monkeypatch.setattr(oracle, attr, bad)
    caught = []
    for pin_name, pin in PINS.items():
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            caught.append(pin_name)
    assert caught, f"no pin detects the planted mistake {name!r}"
