"""Parity of the q6_K x q8_1 variant with the CPU oracle, through the C ABI (needs a GPU).

Bars: repacked bytes equal to the layout reference; the group dot products S (16 values per
group, S = sum q * (u - 32)) bit-exact; C within 1e-5 * T per element, T = sum over groups of
|da * d*sc * S| (float64, from the oracle). Inputs come from synth.py; nothing the GPU
produces feeds the oracle.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_within_tolerance, gpu_quantize, say, to_dev
from tests.layout_ref import repack_q6k_reference

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")

LARGE, SMALL, MEDIUM = mmq.MMQ_TILE_LARGE, mmq.MMQ_TILE_SMALL, mmq.MMQ_TILE_MEDIUM
HALF = mmq.MMQ_TILE_HALF
# (M, K, N, activation kind, x seed, weight kind, w seed)
SHAPES = {
    "tiny": (128, 512, 256, "normal", 1000, "random_fields", 2100),
    "qproj": (2048, 4096, 4096, "normal_outliers", 1001, "fit", 2101),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()


@functools.lru_cache(maxsize=2)
def case(name):
    M, K, N, xk, xs, wk, ws = SHAPES[name]
    x = synth.activations(xk, M, K, xs)
    w, f = synth.q6k_weights(wk, N, K, ws)
    return x, w, f, oracle.quantize_q8_1(x), oracle.decode_q6_K(w)


def gpu_repack6(w, N, K):
    rep = torch.empty(mmq.mmq_q6K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    mmq.repack_q6_K(to_dev(w), N, K, rep)
    torch.cuda.synchronize()
    return rep


def gpu_mmq6(M, N, K, q8, rep, **kw):
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q6K_q8_1_ex(M, N, K, q8, rep, C, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def gpu_dots6(M, N, K, q8, rep, i0, i1, j0, j1, tile=0):
    S = torch.full((K // 16, i1 - i0, j1 - j0), -(2 ** 31), dtype=torch.int32, device="cuda")
    mmq.mmq_q6K_q8_1_blockdots(M, N, K, q8, rep, i0, i1, j0, j1, S, force_tile=tile)
    torch.cuda.synchronize()
    return S.cpu().numpy()


@pytest.mark.parametrize("N,K", [(256, 512), (33, 768), (1, 256), (4096, 4096)])
def test_repack_q6k_bytes(N, K):
    w, f = synth.q6k_weights("random_fields", N, K, N + K)
    say("repack q6_K", N, K)
    got = gpu_repack6(w, N, K).cpu().numpy()
    assert np.array_equal(got, repack_q6k_reference(f))


@pytest.mark.parametrize("tile", [LARGE, SMALL, MEDIUM, HALF])
def test_q6k_group_dots_tiny_every_element(tile):
    x, w, f, q, wo = case("tiny")
    M, K, N = SHAPES["tiny"][:3]
    q8, rep = gpu_quantize(x), gpu_repack6(w, N, K)
    say("q6_K dots tiny", tile)
    S = gpu_dots6(M, N, K, q8, rep, 0, M, 0, N, tile)
    assert np.array_equal(S.astype(np.int64), oracle.block_dots_q6K(q, wo, range(M), range(N)))


@pytest.mark.parametrize("tile", [LARGE, SMALL])
def test_q6k_group_dots_qproj_windows(tile):
    x, w, f, q, wo = case("qproj")
    M, K, N = SHAPES["qproj"][:3]
    q8, rep = gpu_quantize(x), gpu_repack6(w, N, K)
    for (i0, i1, j0, j1) in [(0, 40, 0, 70), (2016, 2048, 4060, 4096), (700, 733, 1000, 1031)]:
        say("q6_K dots qproj", tile, (i0, i1, j0, j1))
        S = gpu_dots6(M, N, K, q8, rep, i0, i1, j0, j1, tile)
        want = oracle.block_dots_q6K(q, wo, range(i0, i1), range(j0, j1))
        assert np.array_equal(S.astype(np.int64), want)


@pytest.mark.parametrize("tile", [0, LARGE, SMALL, MEDIUM, HALF])
def test_q6k_tiny_every_element(tile):
    x, w, f, q, wo = case("tiny")
    M, K, N = SHAPES["tiny"][:3]
    q8, rep = gpu_quantize(x), gpu_repack6(w, N, K)
    say("q6_K mmq tiny", tile)
    C = gpu_mmq6(M, N, K, q8, rep, force_tile=tile)
    C_ref = oracle.mmq_q6K(q, wo)
    _, T = oracle.mmq_q6K_terms(q, wo)
    r = assert_within_tolerance(C, C_ref, T)
    say("max |err|/T", r)


def test_q6k_qproj_every_element():
    x, w, f, q, wo = case("qproj")
    M, K, N = SHAPES["qproj"][:3]
    q8, rep = gpu_quantize(x), gpu_repack6(w, N, K)
    say("q6_K mmq qproj full")
    C = gpu_mmq6(M, N, K, q8, rep)
    assert mmq.mmq_last_kernel()["tile"] == LARGE
    C_terms, T = oracle.mmq_q6K_terms(q, wo)
    C_ref = oracle.mmq_q6K(q, wo)
    assert np.all(np.abs(C_ref - C_terms) <= 1e-12 * T)
    r = assert_within_tolerance(C, C_ref, T)
    say("max |err|/T", r)


def test_q6k_tiles_agree_bitwise():
    x = synth.activations("normal_outliers", 300, 1024, 55)
    w, f = synth.q6k_weights("fit", 200, 1024, 56)
    q8, rep = gpu_quantize(x), gpu_repack6(w, 200, 1024)
    say("q6_K tiles agree")
    a = gpu_mmq6(300, 200, 1024, q8, rep, force_tile=LARGE)
    b = gpu_mmq6(300, 200, 1024, q8, rep, force_tile=SMALL)
    c = gpu_mmq6(300, 200, 1024, q8, rep, force_tile=MEDIUM)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))
    q, wo = oracle.quantize_q8_1(x), oracle.decode_q6_K(w)
    _, T = oracle.mmq_q6K_terms(q, wo)
    assert_within_tolerance(a, oracle.mmq_q6K(q, wo), T)


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (33, 33, 256), (130, 97, 512),
                                   (257, 40, 1280), (128, 4096, 4096)])
def test_q6k_edge_shapes_and_split_k(M, N, K):
    x = synth.activations("normal_outliers", M, K, M + N + K)
    w, f = synth.q6k_weights("random_fields", N, K, M * N + K)
    q8, rep = gpu_quantize(x), gpu_repack6(w, N, K)
    q, wo = oracle.quantize_q8_1(x), oracle.decode_q6_K(w)
    _, T = oracle.mmq_q6K_terms(q, wo)
    C_ref = oracle.mmq_q6K(q, wo)
    ws = torch.empty(4 * M * N * 16 // 4, dtype=torch.float32, device="cuda")
    for kw in ({}, {"force_tile": SMALL}, {"workspace": ws}):
        say("q6_K edge", (M, N, K), list(kw))
        C = gpu_mmq6(M, N, K, q8, rep, **kw)
        assert_within_tolerance(C, C_ref, T)
        say("plan", mmq.mmq_last_kernel()["tile"], mmq.mmq_last_kernel()["splits"])


def test_q6k_integer_case_exact():
    """d = 1, sc = 1, integer activations with a +-127 per block: C = x (u - 32)^T exactly."""
    rng = np.random.default_rng(31)
    M, N, K = 160, 96, 1024
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 5] = rng.choice([-127.0, 127.0], (M, K // 32))
    f = {"d_bits": np.full((N, K // 256), 0x3C00, np.uint16),
         "sc": np.ones((N, K // 16), np.int8),
         "u": rng.integers(0, 64, (N, K), dtype=np.uint8)}
    q8, rep = gpu_quantize(x), gpu_repack6(synth.q6k_pack(f), N, K)
    want = (x.astype(np.int64) @ (f["u"].astype(np.int64) - 32).T).astype(np.float64)
    for tile in (LARGE, SMALL):
        say("q6_K integer case", tile)
        C = gpu_mmq6(M, N, K, q8, rep, force_tile=tile)
        assert np.array_equal(C.astype(np.float64), want)


def test_q6k_refuses_the_few_token_kernels():
    x, w, f, q, wo = case("tiny")
    M, K, N = SHAPES["tiny"][:3]
    q8, rep = gpu_quantize(x), gpu_repack6(w, N, K)
    for tile in (mmq.MMQ_TILE_SKINNY, mmq.MMQ_TILE_GEMV):
        with pytest.raises(mmq.MMQError) as e:
            gpu_mmq6(M, N, K, q8, rep, force_tile=tile)
        assert e.value.status == mmq.MMQ_E_ARG
