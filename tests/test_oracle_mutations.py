"""Planted mistakes in the oracle must make at least one pin fail (CPU only).

Each mutation below is a plausible slip in restating the pages: a wrong rounding
mode or divisor in q8_1, a misread scale packing, swapped nibble halves, a flipped or
dropped term2, a transposed operand. The mistake is planted in the oracle on the CPU
(monkeypatch) and the pins of test_oracle_pins.py are re-run against it.
"""
import numpy as np
import pytest

import oracle
import oracle.mmq_oracle as om
import tests.test_oracle_pins as pins
from tests.conftest import GOLDEN


def _pins():
    return {
        "q8_golden": lambda: pins.test_q8_1_hand_derived_blocks(GOLDEN),
        "q8_invariants": pins.test_q8_1_invariants_random,
        "q4k_golden": lambda: pins.test_q4_K_hand_packed_block(GOLDEN),
        "q4k_roundtrip": pins.test_q4_K_roundtrip_random_fields,
        "q4k_bruteforce": pins.test_q4_K_dequant_bruteforce_reconstruction,
        "int_case": pins.test_mmq_integer_special_case_exact,
        "block_dots": pins.test_block_dots_bruteforce,
        "rational": pins.test_mmq_exact_rational_tiny,
        "direct_vs_terms": pins.test_mmq_direct_equals_term_form,
        "zero_scales": pins.test_mmq_special_case_zero_scales,
    }


def _quantize_variant(x, rounding="away", divisor=127.0, q_from_f16=False, amax_signed=False):
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    xb = x.reshape(M, K // 32, 32)
    amax = xb.max(axis=2) if amax_signed else np.max(np.abs(xb), axis=2)
    d = (amax / np.float32(divisor)).astype(np.float32)
    dq = d.astype(np.float16).astype(np.float32) if q_from_f16 else d
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = np.where(dq > 0, np.float32(1.0) / dq, np.float32(0.0)).astype(np.float32)
        prod = (xb * inv[..., None]).astype(np.float32)
        q = om.round_half_away(prod) if rounding == "away" else np.rint(prod.astype(np.float64))
    q = np.clip(np.where(np.isnan(q), 0.0, q), -127, 127).astype(np.int8)
    return om.Q8(qs=q.reshape(M, K), da_bits=om.f16_encode(d),
                 sa=q.astype(np.int32).sum(axis=2, dtype=np.int32))


def _decode_variant(blocks, swap_hi_scales=False, swap_nibbles=False):
    f = _ORIG["decode"](blocks)
    sc, m, v = f.sc.copy(), f.m.copy(), f.v.copy()
    if swap_hi_scales:
        N, nb = sc.shape
        s3, m3 = sc.reshape(N, nb // 8, 8), m.reshape(N, nb // 8, 8)
        s3[..., 4:], m3[..., 4:] = m3[..., 4:].copy(), s3[..., 4:].copy()
    if swap_nibbles:
        N, K = v.shape
        v4 = v.reshape(N, K // 256, 4, 2, 32)
        v = v4[:, :, :, ::-1, :].reshape(N, K)
    return om.Q4K(d=f.d, dmin=f.dmin, sc=sc, m=m, v=v)


_ORIG = {"decode": om.decode_q4_K, "scales": om.q4_K_scales}


def _scales_flipped(w):
    dsv, dmv = _ORIG["scales"](w)
    return dsv, -dmv


def _scales_no_term2(w):
    dsv, dmv = _ORIG["scales"](w)
    return dsv, np.zeros_like(dmv)


def _block_dots_transposed(q, w, rows, cols):
    qs = q.qs[np.asarray(rows)].astype(np.int64)
    v = w.v[np.asarray(cols)].astype(np.int64)
    R, K = qs.shape
    C = v.shape[0]
    nb = K // 32
    # reverses the element order of the weight block: a transposed/misindexed operand
    return np.einsum("ibk,jbk->bij", qs.reshape(R, nb, 32), v.reshape(C, nb, 32)[:, :, ::-1])


MUTATIONS = {
    "round_half_even": ("quantize_q8_1", lambda x: _quantize_variant(x, rounding="even")),
    "divisor_128": ("quantize_q8_1", lambda x: _quantize_variant(x, divisor=128.0)),
    "q_from_f16_scale": ("quantize_q8_1", lambda x: _quantize_variant(x, q_from_f16=True)),
    "amax_signed": ("quantize_q8_1", lambda x: _quantize_variant(x, amax_signed=True)),
    "scale_bits_misread": ("decode_q4_K", lambda b: _decode_variant(b, swap_hi_scales=True)),
    "nibble_halves_swapped": ("decode_q4_K", lambda b: _decode_variant(b, swap_nibbles=True)),
    "term2_sign_flipped": ("q4_K_scales", _scales_flipped),
    "term2_dropped": ("q4_K_scales", _scales_no_term2),
    "operand_transposed": ("block_dots", _block_dots_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(om, attr, bad)        # calls inside the oracle module
    monkeypatch.setattr(oracle, attr, bad)    # calls through the package namespace
    caught = []
    for pin_name, pin in _pins().items():
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:                # a crash would not be a meaningful detection
            caught.append(pin_name)
    assert caught, f"no pin detects the planted mistake {name!r}"


def test_unmutated_oracle_passes_all_pins():
    for pin_name, pin in _pins().items():
        pin()


# ----------------------------------------------------------------------------- f16 comparator
import oracle.f16_oracle as fo  # noqa: E402
import tests.test_oracle_f16_pins as f16pins  # noqa: E402

_F16_ORIG = {"scales": fo.q4_K_scales, "dequant": fo.dequantize_q4_K_f16}


def _f16_pins():
    return {
        "convert_values": f16pins.test_convert_hand_derived_values,
        "convert_order": f16pins.test_convert_keeps_shape_and_order,
        "dequant_golden": f16pins.test_dequant_hand_packed_block,
        "dequant_int": f16pins.test_dequant_integer_case_exact,
        "dequant_ulp": f16pins.test_dequant_within_one_ulp_of_the_exact_value,
        "gemm_int": f16pins.test_gemm_integer_case_exact,
        "gemm_rational": f16pins.test_gemm_exact_rationals_tiny,
    }


def _dequant_single_rounding(w):
    # rounds the exact value straight to f16 instead of through float32
    return oracle.f16_encode(oracle.dequantize_q4_K(w).astype(np.float16).astype(np.float32))


def _f16_scales_flipped(w):
    dsv, dmv = _F16_ORIG["scales"](w)
    return dsv, -dmv


def _convert_truncating(x):
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    # drop the 13 low significand bits (rounds toward zero for normal values)
    t = (bits & ~np.uint64(0x1FFF)).astype(np.uint32).view(np.float32)
    with np.errstate(over="ignore"):
        return oracle.f16_encode(t)


def _gemm_transposed(a_bits, w_bits):
    a = oracle.f16_decode(a_bits)
    w = oracle.f16_decode(w_bits)[:, ::-1]          # a misindexed K axis of the weights
    return a @ w.T, np.abs(a) @ np.abs(w).T


F16_MUTATIONS = {
    "f16_single_rounding": ("dequantize_q4_K_f16", _dequant_single_rounding),
    "f16_dmv_sign_flipped": ("q4_K_scales", _f16_scales_flipped),
    "f16_convert_truncating": ("convert_f32_f16", _convert_truncating),
    "f16_gemm_operand_transposed": ("gemm_f16", _gemm_transposed),
}


@pytest.mark.parametrize("name", sorted(F16_MUTATIONS))
def test_planted_f16_mistake_is_caught(name, monkeypatch):
    attr, bad = F16_MUTATIONS[name]
    monkeypatch.setattr(fo, attr, bad)
    if hasattr(oracle, attr) and attr != "q4_K_scales":
        monkeypatch.setattr(oracle, attr, bad)
    caught = []
    for pin_name, pin in _f16_pins().items():
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            caught.append(pin_name)
    assert caught, f"no pin detects the planted mistake {name!r}"


def test_unmutated_f16_oracle_passes_all_pins():
    for pin_name, pin in _f16_pins().items():
        pin()
