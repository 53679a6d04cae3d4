"""The test-side layout references agree with the layouts include/mmq.h specifies (CPU only).

These pin the storage forms the GPU parity tests compare bytes against: the repacked weight
records, the q8 buffer's derived planes and its three-piece bfloat16 split. None of this is
the method's arithmetic, which the oracle holds and tests/test_oracle_pins.py pins.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.layout_ref import (bf16_pieces, bf16_value, q8_image, q8_regions, read_repacked,
                              repack_reference)


@pytest.mark.parametrize("N,K", [(32, 256), (33, 512), (70, 768), (5, 256)])
def test_repack_reference_roundtrip(N, K):
    f = synth.q4k_random_fields(N, K, N * 7 + K)
    w = synth.q4k_pack(f)
    rep = repack_reference(w)
    assert rep.size == -(-N // 32) * (K // 256) * 4608       # 4.5 bits per weight
    assert rep.size * 8 == 4.5 * (-(-N // 32) * 32) * K
    got = read_repacked(rep, N, K)
    assert np.array_equal(got["v"], f["v"])
    # the headers are the blocks' own 16 bytes, so they decode to the generator's scales
    blocks = np.concatenate([got["hdr"], np.zeros((N, K // 256, 128), np.uint8)], axis=2)
    dec = oracle.decode_q4_K(blocks)
    assert np.array_equal(dec.d, f["d_bits"].view(np.float16).astype(np.float64))
    assert np.array_equal(dec.dmin, f["dmin_bits"].view(np.float16).astype(np.float64))
    assert np.array_equal(dec.sc, f["sc"].astype(np.int64))
    assert np.array_equal(dec.m, f["m"].astype(np.int64))
    # padding rows of the last tile are zero, nibbles and headers
    nt = -(-N // 32)
    last = rep.reshape(nt, K // 256, 4608)[-1]
    rows_used = N - (nt - 1) * 32
    nib = last[:, :4096].reshape(K // 256, 4, 2, 32, 16)
    assert np.all(nib[:, :, :, rows_used:, :] == 0)
    assert np.all(last[:, 4096:].reshape(K // 256, 32, 16)[:, rows_used:, :] == 0)


def test_repack_reference_nibble_and_header_order():
    """Record byte (g, h, j, e) is q4_K nibble byte 32g + 16h + e of row j; record byte
    4096 + 16j + e is byte e of row j's block."""
    f = synth.q4k_random_fields(32, 512, 1)
    w = synth.q4k_pack(f)
    rep = repack_reference(w)
    for g, h, j, e in [(0, 0, 0, 0), (3, 1, 31, 15), (2, 0, 17, 9), (1, 1, 5, 3)]:
        assert rep[((g * 2 + h) * 32 + j) * 16 + e] == w[j, 0, 16 + 32 * g + 16 * h + e]
    for s, j, e in [(0, 0, 0), (1, 31, 15), (1, 7, 4), (0, 12, 2)]:
        assert rep[s * 4608 + 4096 + 16 * j + e] == w[j, s, e]


# (value, expected pieces) derived by hand from round-to-nearest-even at 8 significant bits
_BF16_PIECE_CASES = [
    (1.0, (0x3F80, 0, 0)),
    (1 + 2.0 ** -8, (0x3F80, 0x3B80, 0)),              # tie, even side is 1.0; rest 2^-8
    (1 + 3 * 2.0 ** -8, (0x3F82, 0xBB80, 0)),          # tie, even side is 1 + 2^-6
    (1 + 2.0 ** -9 + 2.0 ** -17, (0x3F80, 0x3B00, 0x3700)),  # below the tie; the rest is
    (-(1 + 2.0 ** -9 + 2.0 ** -17), (0xBF80, 0xBB00, 0xB700)),  # a tie at 2^-9 (even)
    (0.0, (0, 0, 0)),
    (-0.0, (0x8000, 0, 0)),
    (float("inf"), (0x7F80, 0, 0)),
]


@pytest.mark.parametrize("v,want", _BF16_PIECE_CASES)
def test_bf16_pieces_hand_examples(v, want):
    got = bf16_pieces(np.array([v], np.float32))[0]
    assert tuple(int(g) for g in got) == want


def test_bf16_pieces_exact_for_every_block_factor():
    """p0 + p1 + p2 == v exactly, with shrinking pieces, for da*sa over every sa and f16
    scales spread over the whole f16 range (subnormals included), and for every dmin*m."""
    sa = np.arange(-4064, 4065, dtype=np.float64)
    da = np.arange(1, 0x7C00, 53, dtype=np.uint16).view(np.float16).astype(np.float64)
    v = (da[:, None] * sa[None, :]).ravel()
    dmin = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    v = np.concatenate([v, -(dmin[:, None] * np.arange(64.0)[None, :]).ravel()])
    v32 = v.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), v)        # all exact in float32
    p = bf16_value(bf16_pieces(v32))
    assert np.array_equal(p.sum(axis=-1), v)
    assert np.all(np.abs(p[:, 1]) <= 2.0 ** -8 * np.abs(v) * (1 + 2.0 ** -7))
    assert np.all(np.abs(p[:, 2]) <= 2.0 ** -16 * np.abs(v))


def test_q8_image_layout():
    """Every region of the q8 image, read back by hand from the oracle's q, da and sa."""
    x = synth.activations("normal", 3, 64, 5)
    q = oracle.quantize_q8_1(x)
    img = q8_image(q)
    assert img.dtype == np.uint8 and img.size == 256 + 256 + 48 * 3
    assert np.array_equal(img[:192].view(np.int8).reshape(3, 64), q.qs)
    words = img[192:216].view("<u4").reshape(3, 2)
    assert np.all(img[216:256] == 0)
    pairs = img[256:304].view("<f4").reshape(2, 3, 2)          # [block][row][da, -1.5*2^23*da]
    assert np.all(img[304:512] == 0)
    pieces = bf16_value(img[512:].view("<u2")).reshape(1, 3, 3, 8)   # [sb][piece][row][e]
    assert np.all(pieces[..., 2:] == 0)                        # blocks past K/32
    for i in range(3):
        for b in range(2):
            w = int(words[i, b])
            assert w & 0xFFFF == int(q.da_bits[i, b])
            hi = w >> 16
            sa = hi - 65536 if hi >= 32768 else hi
            assert sa == int(q.sa[i, b])
            da = Fraction(float(np.uint16(w & 0xFFFF).view(np.float16)))
            assert Fraction(float(pairs[b, i, 0])) == da
            assert Fraction(float(pairs[b, i, 1])) == -Fraction(3 * 2 ** 22) * da
            assert sum(Fraction(float(pieces[0, k, i, b])) for k in range(3)) == da * sa
    reg = q8_regions(img, 3, 64)
    assert np.array_equal(reg["qs"], q.qs)
    assert np.array_equal(reg["words"], words)
    assert np.array_equal(reg["pairs"], pairs)


@pytest.mark.parametrize("N,K", [(32, 256), (33, 512), (70, 768), (5, 256)])
def test_repack_q6k_reference_roundtrip(N, K):
    """The q6_K record reference, read back, gives the oracle's decode of the same blocks."""
    from tests.layout_ref import read_repacked_q6k, repack_q6k_reference
    f = synth.q6k_random_fields(N, K, N * 5 + K)
    rep = repack_q6k_reference(f)
    assert rep.size == -(-N // 32) * (K // 256) * 10240
    got = read_repacked_q6k(rep, N, K)
    w = oracle.decode_q6_K(synth.q6k_pack(f))
    assert np.array_equal(got["v"], w.u - 32)
    assert np.array_equal(got["dsv"].astype(np.float64), oracle.q6_K_scales(w))
    nt = -(-N // 32)
    last = rep.reshape(nt, K // 256, 10240)[-1]
    rows_used = N - (nt - 1) * 32
    vals = last[:, :8192].reshape(K // 256, 8, 2, 32, 16)
    assert np.all(vals[:, :, :, rows_used:, :] == 0)
