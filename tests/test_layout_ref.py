"""The test-side repack reference agrees with the layout spec (CPU only)."""
import numpy as np
import pytest

import synth
from tests.layout_ref import read_repacked, repack_reference


@pytest.mark.parametrize("N,K", [(32, 256), (33, 512), (70, 768), (5, 256)])
def test_repack_reference_roundtrip(N, K):
    f = synth.q4k_random_fields(N, K, N * 7 + K)
    rep = repack_reference(synth.q4k_pack(f), f)
    assert rep.size == -(-N // 32) * (K // 256) * 6656
    got = read_repacked(rep, N, K)
    assert np.array_equal(got["v"], f["v"])
    d = np.repeat(f["d_bits"].view(np.float16).astype(np.float64), 8, axis=1)
    dmin = np.repeat(f["dmin_bits"].view(np.float16).astype(np.float64), 8, axis=1)
    assert np.array_equal(got["dsv"].astype(np.float64), d * f["sc"])
    assert np.array_equal(got["dmv"].astype(np.float64), -(dmin * f["m"]))
    # padding rows of the last tile are zero
    nt = -(-N // 32)
    last = rep.reshape(nt, K // 256, 6656)[-1]
    rows_used = N - (nt - 1) * 32
    nib = last[:, :4096].reshape(K // 256, 4, 2, 32, 16)
    assert np.all(nib[:, :, :, rows_used:, :] == 0)


def test_repack_reference_nibble_order():
    """Record byte (g, h, j, e) is q4_K nibble byte 32g + 16h + e of row j."""
    f = synth.q4k_random_fields(32, 256, 1)
    w = synth.q4k_pack(f)
    rep = repack_reference(w, f)
    for g, h, j, e in [(0, 0, 0, 0), (3, 1, 31, 15), (2, 0, 17, 9), (1, 1, 5, 3)]:
        assert rep[((g * 2 + h) * 32 + j) * 16 + e] == w[j, 0, 16 + 32 * g + 16 * h + e]
