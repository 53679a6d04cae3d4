"""Parity at the largest sizes each entry point accepts (needs a GPU with ~90 GB free).

The kernels address operands with 32-bit offsets, or loop with 64-bit indices, and these
cases sit at the edge of what each accepts:
- the integer GEMM at M*K = 2^31 - 4096 (its limit is M*K < 2^31), and at K = 2^24 (its
  limit);
- the f16 GEMM at M*K = 2^30 - 4096 (limit M*K < 2^30);
- the conversion and the dequantization past 2^32 elements (64-bit indices);
- the quantize prepass at M*K = 2^34 - 4096 (its limit is M*K < 2^34).

The large operands are built on the device by repeating a seeded block from synth.py (row r
of the operand is row r mod R of the block). The oracle therefore gets the same values for
any row it checks. Checked rows include the first and the last, where the offsets are
largest.
"""
import numpy as np
import pytest

import oracle
from tests.layout_ref import q8_image
import synth
from tests.gpu_util import assert_within_tolerance, say, to_dev

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def repeat_rows(block: np.ndarray, rows: int) -> "torch.Tensor":
    """Device tensor of `rows` rows: row r is block[r % len(block)]."""
    b = to_dev(block)
    reps = -(-rows // block.shape[0])
    return b.repeat((reps,) + (1,) * (block.ndim - 1))[:rows].contiguous()


def check_rows(M):
    return sorted({0, 1, 4095, 4096, M // 2, M - 129, M - 128, M - 33, M - 2, M - 1})


@pytest.mark.parametrize("tile", [mmq.MMQ_TILE_AUTO, mmq.MMQ_TILE_SMALL])
def test_mmq_largest_activations(tile):
    K, N = 4096, 64
    M = ((1 << 31) - 1) // K                  # M*K = 2^31 - 4096
    block = synth.activations("normal_outliers", 4096, K, 5001)
    w, _ = synth.q4k_weights("fit", N, K, 5002)
    say("mmq largest activations", M, N, K, "tile", tile)
    x = repeat_rows(block, M)
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")
    mmq.quantize_q8_1(x, M, K, q8)
    del x
    rep = torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    mmq.repack_q4_K(to_dev(w), N, K, rep)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_q8_1_ex(M, N, K, q8, rep, C, force_tile=tile)
    torch.cuda.synchronize()
    rows = check_rows(M)
    got = C[rows].cpu().numpy()
    q = oracle.quantize_q8_1(block[[r % 4096 for r in rows]])
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    r = assert_within_tolerance(got, oracle.mmq(q, wo), T)
    say("max |err|/T", r, "plan", mmq.mmq_last_kernel()["tile"])


@pytest.mark.parametrize("M", [2, 16])
def test_mmq_largest_k(M):
    """K at its limit (65536 super-blocks) on every tile; M = 16 takes the decode tile's
    matrix-unit form and the fused call's skinny kernel, M = 2 the vector-ALU form for both."""
    N, K = 33, 1 << 24
    x = synth.activations("normal_outliers", M, K, 5003)
    w, _ = synth.q4k_weights("random_fields", N, K, 5004)
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    C_ref = oracle.mmq(q, wo)
    _, T = oracle.mmq_terms(q, wo)
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")
    rep = torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    say("mmq largest K: quantize, repack", M, N, K)
    mmq.quantize_q8_1(to_dev(x), M, K, q8)
    mmq.repack_q4_K(to_dev(w), N, K, rep)
    out = {}
    for tile in (mmq.MMQ_TILE_SKINNY, mmq.MMQ_TILE_SMALL, mmq.MMQ_TILE_LARGE, mmq.MMQ_TILE_GEMV):
        say("mmq largest K", tile)
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        mmq.mmq_q4K_q8_1_ex(M, N, K, q8, rep, C, force_tile=tile)
        torch.cuda.synchronize()
        out[tile] = C.cpu().numpy()
        r = assert_within_tolerance(out[tile], C_ref, T)
        say("max |err|/T", r)
    # the decode kernel quantizing its own activations: bit for bit the two-step result
    say("mmq_q4K_f32 largest K")
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_f32(M, N, K, to_dev(x), rep, C)
    torch.cuda.synchronize()
    fused = mmq.MMQ_TILE_GEMV if M <= 8 else mmq.MMQ_TILE_SKINNY
    assert mmq.mmq_last_kernel()["tile"] == fused
    assert np.array_equal(C.cpu().numpy().view(np.uint32), out[fused].view(np.uint32))


def test_gemm_f16_largest():
    K, N = 4096, 64
    M = ((1 << 30) - 1) // K                  # M*K = 2^30 - 4096
    a_block = oracle.convert_f32_f16(synth.activations("normal_outliers", 4096, K, 5005))
    rng = np.random.default_rng(5006)
    w_bits = oracle.convert_f32_f16((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    say("gemm_f16 largest", M, N, K)
    a = repeat_rows(a_block.view(np.int16), M)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.gemm_f16(M, N, K, a, to_dev(w_bits.view(np.int16)), C)
    torch.cuda.synchronize()
    rows = check_rows(M)
    got = C[rows].cpu().numpy().astype(np.float64)
    C_ref, T = oracle.gemm_f16(a_block[[r % 4096 for r in rows]], w_bits)
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - C_ref) <= K * 2.0 ** -24 * T)


def test_convert_past_2_32_elements():
    K = 4096
    M = (1 << 20) + 1                         # M*K = 2^32 + 4096 values
    block = synth.activations("normal_outliers", 4096, K, 5007)
    say("convert past 2^32 elements", M, K)
    x = repeat_rows(block, M)
    out = torch.empty(M * K, dtype=torch.int16, device="cuda")
    mmq.convert_f32_f16(x, M, K, out)
    torch.cuda.synchronize()
    del x
    rows = sorted({0, 1, (1 << 20) - 1, 1 << 20, M - 1})
    got = out.view(M, K)[rows].cpu().numpy().view(np.uint16)
    assert np.array_equal(got, oracle.convert_f32_f16(block[[r % 4096 for r in rows]]))


def test_dequantize_past_2_32_weights():
    K = 4096
    N = (1 << 20) + 33                        # N*K past 2^32, ragged last tile
    w_block, _ = synth.q4k_weights("random_fields", 4096, K, 5008)
    say("dequantize past 2^32 weights", N, K)
    w = repeat_rows(w_block, N)
    out = torch.empty(N * K, dtype=torch.int16, device="cuda")
    mmq.dequantize_q4_K_f16(w, N, K, out)
    torch.cuda.synchronize()
    del w
    rows = sorted({0, 1, (1 << 20) - 1, 1 << 20, N - 1})
    got = out.view(N, K)[rows].cpu().numpy().view(np.uint16)
    want = oracle.dequantize_q4_K_f16(oracle.decode_q4_K(w_block[[r % 4096 for r in rows]]))
    assert np.array_equal(got, want)


def q8_rows(image, M: int, K: int, rows):
    """The parts of a q8_1 byte image (uint8, device tensor or numpy) that belong to `rows`:
    int8 values, scale words, (da, -1.5*2^23*da) plane entries and bf16 pieces, as numpy
    arrays."""
    def host(a):
        return a.cpu().numpy() if hasattr(a, "cpu") else np.asarray(a)
    nb, nsb = K // 32, -(-K // 256)
    P = -(-(M * K + 4 * M * nb) // 256) * 256
    Q = -(-(P + 8 * M * nb) // 256) * 256
    qs = np.stack([host(image[r * K:(r + 1) * K]) for r in rows])
    words = np.stack([host(image[M * K + 4 * nb * r:M * K + 4 * nb * (r + 1)]) for r in rows])
    plane = np.stack([host(image[P + 8 * (b * M + r):P + 8 * (b * M + r) + 8])
                      for b in range(nb) for r in rows])
    pieces = np.stack([host(image[Q + 16 * (i * M + r):Q + 16 * (i * M + r) + 16])
                       for i in range(3 * nsb) for r in rows])
    return qs, words, plane, pieces


@pytest.mark.parametrize("K", [4096, 4128])
def test_quantize_largest(K):
    """quantize_q8_1 at M*K just below 2^34, its limit: 64 GiB of f32 input. K = 4096 takes
    the prepass for whole super-blocks, K = 4128 the one for any multiple of 32."""
    M = ((1 << 34) - 1) // K
    R = 1024
    block = synth.activations("normal_outliers", R, K, 5009 + K)
    say("quantize largest", M, K)
    b = to_dev(block)
    x = torch.empty((M, K), dtype=torch.float32, device="cuda")
    full = M // R * R
    x[:full].view(-1, R, K).copy_(b.unsqueeze(0).expand(full // R, R, K))
    x[full:].copy_(b[:M - full])
    del b
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")
    mmq.quantize_q8_1(x, M, K, q8)
    torch.cuda.synchronize()
    del x
    # 16-byte input words past 2^31 from row 2^31 / (K/4) on
    edge = (1 << 31) // (K // 4)
    rows = sorted({0, 1, 31, 32, edge - 1, edge, M // 2, M - 33, M - 32, M - 2, M - 1})
    got = q8_rows(q8, M, K, rows)
    want_image = q8_image(oracle.quantize_q8_1(block[[r % R for r in rows]]))
    want = q8_rows(want_image, len(rows), K, range(len(rows)))
    for name, g, w in zip(("qs", "words", "(da, nda) plane", "pieces"), got, want):
        assert np.array_equal(g, w), f"{name}: {np.count_nonzero(g != w)} bytes differ"
