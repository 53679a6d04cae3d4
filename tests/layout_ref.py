"""Reference byte images of the library's own layouts, written from include/mmq.h.

These are test-side restatements of the documented layouts (they are not the method's
arithmetic, which lives in oracle/): the repacked weight records that repack_q4_K must
produce, and a reader of such records used to check the layout spec round-trips.
"""
import numpy as np

import oracle

TILE_ROWS = 32
TILE_BYTES = 6656


def repack_reference(w_blocks: np.ndarray, fields: dict) -> np.ndarray:
    """Expected repack_q4_K output for GGUF blocks u8 [N, K/256, 144] encoding `fields`."""
    N, nsb, _ = w_blocks.shape
    nt = -(-N // TILE_ROWS)
    pad = nt * TILE_ROWS - N
    wp = np.concatenate([w_blocks, np.zeros((pad, nsb, 144), np.uint8)]) if pad else w_blocks
    out = np.zeros((nt, nsb, TILE_BYTES), np.uint8)
    nib = wp[..., 16:144].reshape(nt, TILE_ROWS, nsb, 4, 2, 16)        # [t, j, s, g, h, 16]
    out[..., :4096] = nib.transpose(0, 2, 3, 4, 1, 5).reshape(nt, nsb, 4096)
    d = fields["d_bits"].view(np.float16).astype(np.float32)           # [N, nsb]
    dmin = fields["dmin_bits"].view(np.float16).astype(np.float32)
    sc = fields["sc"].astype(np.float32).reshape(N, nsb, 8)
    m = fields["m"].astype(np.float32).reshape(N, nsb, 8)
    dsv = np.zeros((nt * TILE_ROWS, nsb, 8), np.float32)
    dmv = np.zeros((nt * TILE_ROWS, nsb, 8), np.float32)
    dsv[:N] = d[..., None] * sc
    dmv[:N] = -(dmin[..., None] * m)
    a = dsv.reshape(nt, TILE_ROWS, nsb, 8).transpose(0, 2, 3, 1)        # [t, s, b, j]
    out[..., 4096:5120] = np.ascontiguousarray(a).view(np.uint8).reshape(nt, nsb, 1024)
    pc = oracle.bf16_pieces(dmv).reshape(nt, TILE_ROWS, nsb, 8, 3)      # [t, j, s, b, i]
    pc = np.ascontiguousarray(pc.transpose(0, 2, 4, 1, 3)).astype("<u2")  # [t, s, i, j, b]
    out[..., 5120:6656] = pc.view(np.uint8).reshape(nt, nsb, 1536)
    return out.reshape(-1)


def read_repacked(rep: np.ndarray, N: int, K: int) -> dict:
    """Decode repacked records back into v [N, K], dsv and dmv [N, K/32] (float32)."""
    nsb = K // 256
    nt = -(-N // TILE_ROWS)
    r = rep.reshape(nt, nsb, TILE_BYTES)
    nib = r[..., :4096].reshape(nt, nsb, 4, 2, TILE_ROWS, 16)          # [t, s, g, h, j, 16]
    lo = nib & 15
    hi = nib >> 4
    v = np.stack([lo, hi], axis=3)                                     # [t, s, g, lohi, h, j, 16]
    v = v.transpose(0, 5, 1, 2, 3, 4, 6).reshape(nt * TILE_ROWS, K)    # [t, j, s, g, lohi, h, e]
    dsv = r[..., 4096:5120].copy().view(np.float32).reshape(nt, nsb, 8, TILE_ROWS)
    dsv = dsv.transpose(0, 3, 1, 2).reshape(nt * TILE_ROWS, K // 32)
    pc = r[..., 5120:6656].copy().view("<u2").reshape(nt, nsb, 3, TILE_ROWS, 8)
    vals = (pc.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dmv = vals.sum(axis=2).transpose(0, 2, 1, 3).reshape(nt * TILE_ROWS, K // 32)
    return {"v": v[:N], "dsv": dsv[:N], "dmv": dmv[:N]}
