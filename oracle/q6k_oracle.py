"""Plain CPU oracle of the q6_K x q8_1 MMQ variant (test infrastructure, like the rest of oracle/).

Page cited (title as published):
  [r16] "21 · r16 — Narrow kernel gets the rank-1 fold (LANDED)": the rank-1 fold of the
        activation block sums was later carried over to the q6_K kernel family (§2.3, §5).

The pages name q6_K but give neither its byte layout nor its arithmetic. The reading taken
here is the GGUF q6_K format, restated in prose in decode_q6_K: 256 values per super-block,
each a 6-bit unsigned u whose quantized weight is the signed integer u - 32, one int8 scale
sc per 16 consecutive values and one f16 scale d per super-block, so that

    w_jk = d_j * sc_{j,g(k)} * (u_jk - 32),          g(k) = k // 16.

Against q8_1 activations (blocks of 32, scale da, integer sum sa) the product is

    C_ij = sum_k (da_{i,b(k)} q_ik) w_jk = sum_g da_{i,b(g)} * (d_j sc_jg) * S_ijg,
    S_ijg = sum_{k in g} q_ik (u_jk - 32)                (the integer block dot product),

one term per 16-value group: q6_K has no min, so the two-term rescale of q4_K has only its
first term. The pages' fold form computes the same thing from the unsigned values and a
rank-1 correction, S_ijg = sum_{k in g} q_ik u_jk - 32 * sa16_ig with sa16 the integer sum
of the activation values of group g; mmq_q6K_fold_terms restates that form and the pins
check that both agree exactly.

Parity status: every function is pinned by tests/test_oracle_q6k_pins.py (a hand-packed
block, brute-force reconstruction, an exact integer case, the fold identity, planted
mistakes). No function is "parity unpinned".
"""
from __future__ import annotations

from typing import NamedTuple, Sequence

import numpy as np
from numpy.typing import NDArray

from .mmq_oracle import Q8, QK8, f16_decode

QK_K = 256
Q6K_BLOCK_BYTES = 210
GROUP = 16            # values per q6_K scale


class Q6K(NamedTuple):
    """Decoded q6_K fields."""
    d: NDArray        # float64 [N, K/256]  super-block scale (an f16 value)
    sc: NDArray       # int64 [N, K/16]     int8 scale of each group of 16 values
    u: NDArray        # int64 [N, K]        unsigned 6-bit values 0..63 (weight value u - 32)


def decode_q6_K(blocks) -> Q6K:
    """Decode q6_K super-blocks u8 [N, K/256, 210] into their fields.

    The GGUF q6_K layout: a super-block holds 256 values in two halves of 128. Value
    128h + 32q + l (h = 0..1, q = 0..3, l = 0..31):
      - low 4 bits: byte 64h + l + 32*(q mod 2) of bytes 0..127, its low nibble when q < 2
        and its high nibble when q >= 2;
      - high 2 bits: bits 2q, 2q+1 of byte 128 + 32h + l (bytes 128..191);
    bytes 192..207 are the 16 scales as int8, scale g for values 16g..16g+15; bytes 208..209
    are d as a little-endian f16.
    """
    blk = np.asarray(blocks, dtype=np.uint8)
    N, nsb, nbytes = blk.shape
    if nbytes != Q6K_BLOCK_BYTES:
        raise ValueError("q6_K blocks must be 210 bytes")
    ql = blk[..., 0:128].astype(np.int64).reshape(N, nsb, 2, 64)     # [n, s, half, byte]
    qh = blk[..., 128:192].astype(np.int64).reshape(N, nsb, 2, 32)
    u = np.empty((N, nsb, 2, 4, 32), dtype=np.int64)                 # [n, s, half, q, l]
    for q in range(4):
        low_byte = ql[..., 32 * (q % 2): 32 * (q % 2) + 32]
        low = (low_byte & 15) if q < 2 else (low_byte >> 4)
        high = (qh >> (2 * q)) & 3
        u[:, :, :, q, :] = low | (high << 4)
    sc = blk[..., 192:208].copy().view(np.int8).astype(np.int64)     # [n, s, 16]
    d = f16_decode(np.ascontiguousarray(blk[..., 208:210]).view("<u2")[..., 0])
    return Q6K(d=d, sc=sc.reshape(N, nsb * 16), u=u.reshape(N, nsb * QK_K))


def q6_K_scales(w: Q6K) -> NDArray:
    """Per group of 16 the effective scale dsv = d * sc (exact in float64) [N, K/16]."""
    return np.repeat(w.d, QK_K // GROUP, axis=1) * w.sc


def dequantize_q6_K(w: Q6K) -> NDArray:
    """Weights as float64 [N, K]: d * sc * (u - 32), exact in float64."""
    dsv = q6_K_scales(w)
    N, K = w.u.shape
    v = (w.u - 32).reshape(N, K // GROUP, GROUP).astype(np.float64)
    return (dsv[..., None] * v).reshape(N, K)


def mmq_q6K(q: Q8, w: Q6K, rows: Sequence[int] | None = None) -> NDArray:
    """C[i, j] = sum_k (da_i,b(k) * q_ik) * w_jk in float64: dequantize both operands and take
    one f64 matrix product (every product exact, the sum correct to ~1e-15 relative)."""
    if rows is None:
        rows = np.arange(q.qs.shape[0])
    qs = q.qs[rows].astype(np.float64)
    da = f16_decode(q.da_bits[rows])
    R, K = qs.shape
    a = (qs.reshape(R, K // QK8, QK8) * da[..., None]).reshape(R, K)
    return a @ dequantize_q6_K(w).T


def block_dots_q6K(q: Q8, w: Q6K, rows: Sequence[int], cols: Sequence[int]) -> NDArray:
    """S[g, i, j] = sum_{k in group g} q_ik * (u_jk - 32), exact int64 by brute force;
    shape [K/16, len(rows), len(cols)]."""
    qs = q.qs[np.asarray(rows)].astype(np.int64)
    v = w.u[np.asarray(cols)].astype(np.int64) - 32
    R, K = qs.shape
    ng = K // GROUP
    return np.einsum("igk,jgk->gij", qs.reshape(R, ng, GROUP), v.reshape(v.shape[0], ng, GROUP))


def mmq_q6K_terms(q: Q8, w: Q6K, rows: Sequence[int] | None = None):
    """The per-group form of C and the tolerance scale T, both float64:

        C_terms[i, j] = sum_g da_{i,b(g)} * dsv_jg * S_ijg,   T = sum_g |da * dsv * S|

    with S the signed integer group dot products, formed one group at a time as an f64
    product of integer matrices (exact). Returns (C_terms, T), [R, N]."""
    if rows is None:
        rows = np.arange(q.qs.shape[0])
    rows = np.asarray(rows)
    qs = q.qs[rows].astype(np.float64)
    R, K = qs.shape
    da = f16_decode(q.da_bits[rows])                   # [R, K/32]
    dsv = q6_K_scales(w)                               # [N, K/16]
    v = (w.u - 32).astype(np.float64)
    C = np.zeros((R, w.u.shape[0]))
    T = np.zeros_like(C)
    for g in range(K // GROUP):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        t = qs[:, ks] @ v[:, ks].T                     # S, exact integers
        t *= da[:, g // 2: g // 2 + 1]
        t *= dsv[None, :, g]
        C += t
        np.abs(t, out=t)
        T += t
    return C, T


def mmq_q6K_fold_terms(q: Q8, w: Q6K, rows: Sequence[int] | None = None) -> NDArray:
    """The fold form [r16 §2.3]: from the unsigned values, term1 = da*dsv*sum q*u per group,
    plus the rank-1 correction of the offset, term2 = (-32 dsv_jg) * (da * sa16_ig), with sa16
    the integer sum of the group's 16 activation values. Returns C [R, N] in float64."""
    if rows is None:
        rows = np.arange(q.qs.shape[0])
    rows = np.asarray(rows)
    qs = q.qs[rows].astype(np.float64)
    R, K = qs.shape
    da = f16_decode(q.da_bits[rows])
    dsv = q6_K_scales(w)
    u = w.u.astype(np.float64)
    ng = K // GROUP
    sa16 = qs.reshape(R, ng, GROUP).sum(axis=2)        # integer group sums
    da_g = np.repeat(da, 2, axis=1)                    # the token scale of each group
    C = (da_g * sa16) @ (-32.0 * dsv).T                # sum_g term2, one f64 product
    for g in range(ng):
        ks = slice(g * GROUP, (g + 1) * GROUP)
        t = qs[:, ks] @ u[:, ks].T
        t *= da_g[:, g:g + 1]
        t *= dsv[None, :, g]
        C += t
    return C
