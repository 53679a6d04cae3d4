"""Plain CPU oracle of the q4_K x q8_1 MMQ (test infrastructure; see the package docstring).

Pages cited (titles as published):
  [r15] "20 · r15 — f32-accumulate mma probe (dead end) + rank-1 term2 rescale (LANDED)"
  [r16] "21 · r16 — Narrow kernel gets the rank-1 fold (LANDED)"
  [r12] "16 · r12 — 16-chain warp tile + ldmatrix (LANDED)"

Where the pages leave a step open the plainest reading is taken; each such reading
is named in the docstring of the function that takes it.

Parity status: every function here is pinned by tests/test_oracle_pins.py against
closed forms, hand-derived fixtures (tests/golden/), brute force on tiny inputs or
an exact integer special case. No function is "parity unpinned".
"""
from __future__ import annotations

from typing import NamedTuple, Sequence

import numpy as np
from numpy.typing import NDArray

QK8 = 32              # q8_1 block length: activations are quantized in blocks of 32 [r15 §2.1]
QK_K = 256            # q4_K super-block length (8 sub-blocks of 32) [r12 §2, "KDR=4 restage-skip"]
Q4K_BLOCK_BYTES = 144  # 2+2 bytes f16 d/dmin, 12 bytes 6-bit sc/m, 128 bytes of nibbles


class Q8(NamedTuple):
    """q8_1 activations: per 32-block an f16 scale da and the integer block sum sa."""
    qs: NDArray       # int8  [M, K]
    da_bits: NDArray  # uint16 [M, K/32], f16 bit pattern of the block scale
    sa: NDArray       # int32 [M, K/32], integer sum of the block's 32 quantized values


class Q4K(NamedTuple):
    """Decoded q4_K fields."""
    d: NDArray     # float64 [N, K/256]  super-block scale (an f16 value)
    dmin: NDArray  # float64 [N, K/256]  super-block min scale (an f16 value)
    sc: NDArray    # int64 [N, K/32]     6-bit sub-block scale
    m: NDArray     # int64 [N, K/32]     6-bit sub-block min
    v: NDArray     # int64 [N, K]        4-bit unsigned values 0..15


# ----------------------------------------------------------------------------- float16
def f16_encode(x) -> NDArray:
    """f32 -> f16 bit pattern, IEEE round-to-nearest-even with subnormals (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_decode(bits) -> NDArray:
    """f16 bit pattern -> exact float64 value."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def round_half_away(v) -> NDArray:
    """Round to the nearest integer, ties away from zero (C's roundf), as float64.

    Evaluated in float64, where |v| + 0.5 is exact for every float32 |v| < 2^29.
    """
    v = np.asarray(v, dtype=np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


# ----------------------------------------------------------------------------- q8_1
def quantize_q8_1(x) -> Q8:
    """Quantize f32 activations [M, K] into q8_1 blocks of 32 [r15 §2.1; r16 §3.2].

    The pages define the outputs: int8 values, the block scale da (stored as f16) and the
    in-block integer sum sa, produced by the quantize prepass. They leave the rounding open;
    the reading taken here, for every block x_0..x_31 (float32 throughout):
        amax = max |x_k|
        d    = amax / 127                      (IEEE division, round to nearest)
        id   = 1 / d if d > 0 else 0
        q_k  = round_half_away(x_k * id), clamped to [-127, 127]; a NaN product
               (0 * inf, only when 1/d overflows for a block of tiny values) gives 0
        sa   = sum_k q_k                       (integer; |sa| <= 4064)
        da   = f16(d)                          (round to nearest even)
    q is computed from the f32 d, not from the rounded f16 da.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    if K % QK8:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(M, K // QK8, QK8)
    amax = np.max(np.abs(xb), axis=2)                                   # f32
    d = (amax / np.float32(127.0)).astype(np.float32)                   # f32, RN
    with np.errstate(divide="ignore", over="ignore"):
        inv = np.where(d > 0, np.float32(1.0) / d, np.float32(0.0)).astype(np.float32)
    with np.errstate(invalid="ignore", over="ignore"):
        prod = (xb * inv[..., None]).astype(np.float32)                 # f32, RN
        q = round_half_away(prod)
    q = np.where(np.isnan(q), 0.0, q)
    q = np.clip(q, -127.0, 127.0).astype(np.int8)
    sa = q.astype(np.int32).sum(axis=2, dtype=np.int32)
    return Q8(qs=q.reshape(M, K), da_bits=f16_encode(d), sa=sa)


def decode_q4_K(blocks) -> Q4K:
    """Decode q4_K super-blocks u8 [N, K/256, 144] into their fields [r15 §2.1].

    The pages name the fields (f16 d and dmin per super-block, 6-bit sc and m per 32-k
    sub-block read with "get_scale_min_k4 table semantics", unsigned nibbles 0..15) but
    not the bit packing. The GGUF q4_K layout is read here:
      bytes 0..1 d, 2..3 dmin (f16 little endian); bytes 4..15 the 12 scale bytes s[0..11];
      for sub-block b < 4:  sc = s[b] & 63,   m = s[b+4] & 63
      for sub-block b >= 4: sc = (s[b+4] & 15) | ((s[b-4] >> 6) << 4)
                            m  = (s[b+4] >> 4) | ((s[b]   >> 6) << 4)
      bytes 16..143: group g = 0..3 of 32 bytes; byte t holds element t of sub-block 2g in
      its low nibble and element t of sub-block 2g+1 in its high nibble.
    """
    blk = np.asarray(blocks, dtype=np.uint8)
    N, nsb, nbytes = blk.shape
    if nbytes != Q4K_BLOCK_BYTES:
        raise ValueError("q4_K blocks must be 144 bytes")
    d = f16_decode(np.ascontiguousarray(blk[..., 0:2]).view("<u2")[..., 0])
    dmin = f16_decode(np.ascontiguousarray(blk[..., 2:4]).view("<u2")[..., 0])
    s = blk[..., 4:16].astype(np.int64)
    sc = np.empty((N, nsb, 8), dtype=np.int64)
    m = np.empty((N, nsb, 8), dtype=np.int64)
    for b in range(8):
        if b < 4:
            sc[..., b] = s[..., b] & 63
            m[..., b] = s[..., b + 4] & 63
        else:
            sc[..., b] = (s[..., b + 4] & 15) | ((s[..., b - 4] >> 6) << 4)
            m[..., b] = (s[..., b + 4] >> 4) | ((s[..., b] >> 6) << 4)
    qs = blk[..., 16:144].reshape(N, nsb, 4, 32).astype(np.int64)
    v = np.empty((N, nsb, 8, 32), dtype=np.int64)
    for g in range(4):
        v[:, :, 2 * g, :] = qs[:, :, g, :] & 15
        v[:, :, 2 * g + 1, :] = qs[:, :, g, :] >> 4
    return Q4K(d=d, dmin=dmin, sc=sc.reshape(N, nsb * 8), m=m.reshape(N, nsb * 8),
               v=v.reshape(N, nsb * QK_K))


def q4_K_scales(w: Q4K) -> tuple[NDArray, NDArray]:
    """Per sub-block effective scale dsv = d*sc and negative bias dmv = -(dmin*m) [r15 §2.1].

    Both products are exact in float64 (f16 value times a 6-bit integer).
    """
    d = np.repeat(w.d, 8, axis=1)
    dmin = np.repeat(w.dmin, 8, axis=1)
    return d * w.sc, -(dmin * w.m)


def dequantize_q4_K(w: Q4K, rows: Sequence[int] | None = None) -> NDArray:
    """Weights as float64 [N, K]: b = dsv*v + dmv = d*sc*v - dmin*m [r15 §2.1]. Exact in f64."""
    dsv, dmv = q4_K_scales(w)
    v = w.v if rows is None else w.v[rows]
    if rows is not None:
        dsv, dmv = dsv[rows], dmv[rows]
    N, K = v.shape
    vb = v.reshape(N, K // QK8, QK8).astype(np.float64)
    return (dsv[..., None] * vb + dmv[..., None]).reshape(N, K)


# ----------------------------------------------------------------------------- the product
def _a_f64(q: Q8, rows) -> NDArray:
    """Dequantized activations da*q as float64 (exact: an f16 value times an 8-bit integer)."""
    qs = q.qs[rows].astype(np.float64)
    da = f16_decode(q.da_bits[rows])
    R, K = qs.shape
    return (qs.reshape(R, K // QK8, QK8) * da[..., None]).reshape(R, K)


def mmq(q: Q8, w: Q4K, rows: Sequence[int] | None = None) -> NDArray:
    """C[i, j] = sum_k (da_i,b(k) * q_ik) * w_jk in float64 -- the direct dot product.

    Dequantize both operands to float and take their product with one f64 matrix
    multiply. Every product is exact in f64 and the sum is correct to ~1e-15 relative.
    `rows` selects output rows (all when None); the result is [len(rows), N].
    """
    if rows is None:
        rows = np.arange(q.qs.shape[0])
    a = _a_f64(q, rows)
    wt = dequantize_q4_K(w)
    return a @ wt.T


def block_dots(q: Q8, w: Q4K, rows: Sequence[int], cols: Sequence[int]) -> NDArray:
    """Per-block integer dot products S[b, i, j] = sum_{k in block b} q_ik * v_jk [r15 §2.1].

    Exact int64 by brute force (np.einsum on integers); shape [K/32, len(rows), len(cols)].
    """
    qs = q.qs[np.asarray(rows)].astype(np.int64)
    v = w.v[np.asarray(cols)].astype(np.int64)
    R, K = qs.shape
    C = v.shape[0]
    nb = K // QK8
    return np.einsum("ibk,jbk->bij", qs.reshape(R, nb, QK8), v.reshape(C, nb, QK8))


def mmq_terms(q: Q8, w: Q4K, rows: Sequence[int] | None = None):
    """Two-term rescale form of C and the tolerance scale T, both float64 [r15 §2.1; r16 §2.1].

        C_terms[i, j] = sum_b ( da_ib * dsv_jb * S_ijb  +  dmv_jb * (da_ib * sa_ib) )
        T[i, j]       = sum_b ( |da_ib * dsv_jb * S_ijb| + |dmv_jb * da_ib * sa_ib| )

    term1 scales the integer block dot product S, term2 is the rank-1 correction from the
    block sums sa (the row factor da*sa times the column factor dmv). Each term is exact in
    f64. S is formed one block at a time as an f64 matrix product of integer matrices
    (exact: every partial sum is an integer below 2^16). Summed over b, term2 is the
    product of the [R, K/32] row factors and the [N, K/32] column factors, taken as one f64
    matrix product (and likewise for its absolute values in T). Returns (C_terms, T), [R, N].
    """
    if rows is None:
        rows = np.arange(q.qs.shape[0])
    rows = np.asarray(rows)
    qs = q.qs[rows].astype(np.float64)
    R, K = qs.shape
    nb = K // QK8
    da = f16_decode(q.da_bits[rows])                    # [R, nb]
    sa = q.sa[rows].astype(np.float64)                  # [R, nb]
    dsv, dmv = q4_K_scales(w)                           # [N, nb]
    v = w.v.astype(np.float64)
    dma = da * sa                                       # row factor of term2, exact
    C = dma @ dmv.T                                     # sum_b term2
    T = np.abs(dma) @ np.abs(dmv).T                     # sum_b |term2|
    for b in range(nb):
        ks = slice(b * QK8, (b + 1) * QK8)
        t1 = qs[:, ks] @ v[:, ks].T                     # S, [R, N], exact integers
        t1 *= da[:, b:b + 1]
        t1 *= dsv[None, :, b]                           # term1 = da * dsv * S
        C += t1
        np.abs(t1, out=t1)
        T += t1
    return C, T
