"""Reference byte images of the library's own storage layouts, written from include/mmq.h.

These are test-side restatements of the documented layouts, not the method's arithmetic
(that lives in oracle/, which knows only the q8_1 fields q, da, sa and the q4_K and q6_K
fields).
Each image is built from the oracle's fields:
  - q8_image: the whole q8 buffer quantize_q8_1 writes: q and the packed (da, sa) words,
    then the GEMM's planes derived from da and sa;
  - repack_reference: the repacked weight records repack_q4_K writes (the GGUF blocks'
    bytes regrouped);
  - read_repacked: a reader of such records, used to check that the layout round-trips;
  - repack_q6k_reference, read_repacked_q6k: the same for repack_q6_K;
  - bf16_pieces: the three-piece bfloat16 split of the q8 buffer's piece plane.
"""
import numpy as np

import oracle

TILE_ROWS = 32
TILE_BYTES = 4608
BIAS = 1.5 * 2.0 ** 23  # the GEMM's integer results come offset by this value


def _rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> the float32 bits of its nearest bfloat16 (ties to even), low half zero."""
    b = x.view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)


def bf16_pieces(v) -> np.ndarray:
    """Three bfloat16 values summing exactly to each float32 v, as uint16 bits [..., 3].

    As the header defines them: p0 = bf16_rne(v), p1 = bf16_rne(v - p0), p2 = v - p0 - p1
    (both differences are exact in float32); a non-finite v is stored as {top 16 bits, 0, 0}.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    with np.errstate(invalid="ignore", over="ignore"):   # non-finite v: replaced below
        a = _rne_bf16_bits(v)
        r = (v - a.view(np.float32)).astype(np.float32)
        b = _rne_bf16_bits(r)
        c = (r - b.view(np.float32)).astype(np.float32)
    out = np.stack([a >> 16, b >> 16, c.view(np.uint32) >> 16], axis=-1).astype(np.uint16)
    bad = ~np.isfinite(v)
    out[bad] = 0
    out[bad, 0] = (v[bad].view(np.uint32) >> 16).astype(np.uint16)
    return out


def bf16_value(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _pad256(a: np.ndarray) -> np.ndarray:
    return np.concatenate([a, np.zeros((-a.size) % 256, np.uint8)])


def q8_words(q: oracle.Q8) -> np.ndarray:
    """The packed scale words [M][K/32]: f16 bits of da in bits 0..15, sa (s16) in 16..31."""
    return (q.da_bits.astype(np.uint32)
            | ((q.sa.astype(np.int32) & 0xFFFF).astype(np.uint32) << np.uint32(16)))


def q8_image(q: oracle.Q8) -> np.ndarray:
    """Byte image of a q8 buffer (unwritten padding as zero) from the oracle's q, da, sa.

    Regions: q int8 [M][K]; the scale words [M][K/32]; at the next 256-byte boundary the
    float32 pairs (da, -1.5*2^23*da) [K/32][M]; at the next one the bf16 pieces of da*sa,
    [ceil(K/256)][3][M][8] (piece i of row r, block 8s+e at [s][i][r][e]).
    """
    M, K = q.qs.shape
    nb = K // 32
    nsb = -(-nb // 8)
    head = np.concatenate([q.qs.reshape(-1).view(np.uint8),
                           q8_words(q).astype("<u4").reshape(-1).view(np.uint8)])
    da = oracle.f16_decode(q.da_bits)                           # exact
    dma = da * q.sa.astype(np.float64)                          # exact in float32
    assert np.array_equal(dma.astype(np.float32).astype(np.float64), dma)
    pairs = np.stack([da.T, -BIAS * da.T], axis=-1).astype("<f4")   # [K/32][M][2], exact
    assert np.array_equal(pairs[..., 1].astype(np.float64), -BIAS * da.T)
    pieces = np.zeros((nsb, 3, M, 8), "<u2")
    pc = bf16_pieces(dma.astype(np.float32))                    # [M][K/32][3]
    for b in range(nb):
        pieces[b // 8, :, :, b % 8] = pc[:, b, :].T
    return np.concatenate([_pad256(head), _pad256(pairs.reshape(-1).view(np.uint8)),
                           pieces.reshape(-1).view(np.uint8)])


def q8_regions(img: np.ndarray, M: int, K: int) -> dict:
    """Split a q8 buffer image into its regions: qs, words, pairs (f32), pieces (u16)."""
    nb = K // 32
    P = -(-(M * K + 4 * M * nb) // 256) * 256
    Q = -(-(P + 8 * M * nb) // 256) * 256
    return {"qs": img[:M * K].view(np.int8).reshape(M, K),
            "words": img[M * K:M * K + 4 * M * nb].view("<u4").reshape(M, nb),
            "pairs": img[P:P + 8 * M * nb].view("<f4").reshape(nb, M, 2),
            "pieces": img[Q:].view("<u2").reshape(-1, 3, M, 8)}


def repack_reference(w_blocks: np.ndarray) -> np.ndarray:
    """Expected repack_q4_K output for GGUF blocks u8 [N, K/256, 144]: per (32-row tile,
    super-block) the nibble bytes regrouped [g][h][j][16], then each row's 16-byte header."""
    N, nsb, _ = w_blocks.shape
    nt = -(-N // TILE_ROWS)
    pad = nt * TILE_ROWS - N
    wp = np.concatenate([w_blocks, np.zeros((pad, nsb, 144), np.uint8)]) if pad else w_blocks
    out = np.zeros((nt, nsb, TILE_BYTES), np.uint8)
    nib = wp[..., 16:144].reshape(nt, TILE_ROWS, nsb, 4, 2, 16)        # [t, j, s, g, h, 16]
    out[..., :4096] = nib.transpose(0, 2, 3, 4, 1, 5).reshape(nt, nsb, 4096)
    hdr = wp[..., :16].reshape(nt, TILE_ROWS, nsb, 16)                  # [t, j, s, 16]
    out[..., 4096:] = hdr.transpose(0, 2, 1, 3).reshape(nt, nsb, 512)
    return out.reshape(-1)


def read_repacked(rep: np.ndarray, N: int, K: int) -> dict:
    """Decode repacked records back into the nibble values v [N, K] and the GGUF blocks'
    16-byte headers [N, K/256, 16]."""
    nsb = K // 256
    nt = -(-N // TILE_ROWS)
    r = rep.reshape(nt, nsb, TILE_BYTES)
    nib = r[..., :4096].reshape(nt, nsb, 4, 2, TILE_ROWS, 16)          # [t, s, g, h, j, 16]
    lo = nib & 15
    hi = nib >> 4
    v = np.stack([lo, hi], axis=3)                                     # [t, s, g, lohi, h, j, 16]
    v = v.transpose(0, 5, 1, 2, 3, 4, 6).reshape(nt * TILE_ROWS, K)    # [t, j, s, g, lohi, h, e]
    hdr = r[..., 4096:].reshape(nt, nsb, TILE_ROWS, 16).transpose(0, 2, 1, 3)
    return {"v": v[:N], "hdr": hdr.reshape(nt * TILE_ROWS, nsb, 16)[:N]}


TILE6_BYTES = 10240


def repack_q6k_reference(fields: dict) -> np.ndarray:
    """Expected repack_q6_K output for the q6_K fields (u [N, K], sc [N, K/16], d_bits)."""
    u = np.asarray(fields["u"], np.int64)
    N, K = u.shape
    nsb = K // 256
    nt = -(-N // TILE_ROWS)
    vals = np.zeros((nt * TILE_ROWS, K), np.int64)
    vals[:N] = u - 32
    v = vals.reshape(nt, TILE_ROWS, nsb, 8, 2, 16)                    # [t, j, s, b, h, e]
    v = v.transpose(0, 2, 3, 4, 1, 5).astype(np.int8)                 # [t, s, b, h, j, e]
    d = np.asarray(fields["d_bits"], np.uint16).view(np.float16).astype(np.float32)
    dsv = np.zeros((nt * TILE_ROWS, nsb, 16), np.float32)
    dsv[:N] = d[..., None] * np.asarray(fields["sc"], np.float32).reshape(N, nsb, 16)
    dsv = dsv.reshape(nt, TILE_ROWS, nsb, 16).transpose(0, 2, 3, 1)   # [t, s, g, j]
    out = np.zeros((nt, nsb, TILE6_BYTES), np.uint8)
    out[..., :8192] = np.ascontiguousarray(v).view(np.uint8).reshape(nt, nsb, 8192)
    out[..., 8192:] = np.ascontiguousarray(dsv).view(np.uint8).reshape(nt, nsb, 2048)
    return out.reshape(-1)


def read_repacked_q6k(rep: np.ndarray, N: int, K: int) -> dict:
    """Decode repacked q6_K records back into the values u - 32 [N, K] and dsv [N, K/16]."""
    nsb = K // 256
    nt = -(-N // TILE_ROWS)
    r = rep.reshape(nt, nsb, TILE6_BYTES)
    v = r[..., :8192].copy().view(np.int8).reshape(nt, nsb, 8, 2, TILE_ROWS, 16)
    v = v.transpose(0, 4, 1, 2, 3, 5).reshape(nt * TILE_ROWS, K)      # [t, j, s, b, h, e]
    dsv = r[..., 8192:].copy().view(np.float32).reshape(nt, nsb, 16, TILE_ROWS)
    dsv = dsv.transpose(0, 3, 1, 2).reshape(nt * TILE_ROWS, K // 16)
    return {"v": v[:N].astype(np.int64), "dsv": dsv[:N]}
