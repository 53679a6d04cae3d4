"""Plain CPU oracle of the f16 comparator path (test infrastructure, like the rest of oracle/).

The comparator is the f16 default prefill path that the pages measure the integer product
against: the r15 page ("20 · r15 — f32-accumulate mma probe (dead end) + rank-1 term2
rescale (LANDED)", §5) and the r12 page ("16 · r12 — 16-chain warp tile + ldmatrix
(LANDED)", §1 and §5). Its dequantize step is dq_f16 of the audit page "Round 31 Track C
Audit: dq_f16 (dense_mm.metal) & DW<F> (mma.metal)", §1-2: quantized weights in, an f16
weight matrix out. The pages give no arithmetic for it beyond the q4_K weight formula of the
r15 page (§2.1); the readings taken are named in each docstring.

Parity status: every function is pinned by tests/test_oracle_f16_pins.py (hand-derived
values in tests/golden/q4_K_f16_dequant.json, exact integer special cases, the one-ulp bound
against exact rationals). No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np
from numpy.typing import NDArray

from .mmq_oracle import Q4K, QK8, f16_decode, f16_encode, q4_K_scales


def convert_f32_f16(x) -> NDArray:
    """f32 activations [M, K] -> f16 bit patterns [M, K], nearest value, ties to even.

    Reading: the pages name the f16 path without its conversion; the plainest one is IEEE
    round-to-nearest-even with subnormals and overflow to infinity (f16_encode).
    """
    with np.errstate(over="ignore"):   # overflow to infinity is the defined result
        return f16_encode(np.asarray(x, dtype=np.float32))


def dequantize_q4_K_f16(w: Q4K) -> NDArray:
    """q4_K weights -> f16 bit patterns [N, K]: w = dsv*v + dmv per sub-block [r15 §2.1].

    Reading: the value is evaluated in float32 and then rounded to f16 (nearest, ties to
    even). dsv = d*sc and dmv = -(dmin*m) are exact in float32 (an f16 value times a 6-bit
    integer), and so is dsv*v (at most 21 significant bits); the sum is rounded once to
    float32, then to f16. Where the float32 sum lands on a tie of two f16 values this can
    differ from rounding the exact value straight to f16; the reading fixes the two-step one.
    """
    dsv, dmv = q4_K_scales(w)                                  # f64 [N, K/32], exact
    N, K = w.v.shape
    v = w.v.reshape(N, K // QK8, QK8).astype(np.float32)
    prod = dsv.astype(np.float32)[..., None] * v               # exact in float32
    val = prod + dmv.astype(np.float32)[..., None]             # one float32 rounding
    assert val.dtype == np.float32
    return f16_encode(val.reshape(N, K))


def gemm_f16(a_bits, w_bits) -> tuple[NDArray, NDArray]:
    """C[i, j] = sum_k a_ik * w_jk for f16 operands, and T[i, j] = sum_k |a_ik * w_jk|.

    a_bits [M, K] and w_bits [N, K] are f16 bit patterns. Each product of two f16 values is
    exact in float64 (22 significant bits); the sums are one f64 matrix product each, correct
    to ~K * 2^-53 of T. Returns (C, T), float64 [M, N].
    """
    a = f16_decode(a_bits)
    w = f16_decode(w_bits)
    return a @ w.T, np.abs(a) @ np.abs(w).T
