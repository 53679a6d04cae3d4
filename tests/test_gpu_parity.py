"""Parity of the HIP path with the CPU oracle, through the C ABI (needs a gfx950 GPU).

Bars: q8_1 bytes and per-block integer dot products S bit-exact; f32 outputs within
1e-5 * T per element, T = sum over blocks of |term1| + |term2| (float64, from the oracle).
The GPU path runs end to end (quantize_q8_1 -> repack_q4_K -> mmq_q4K_q8_1) on the same
seeded inputs the oracle gets from synth.py; nothing the GPU produces feeds the oracle.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (assert_within_tolerance, gpu_blockdots, gpu_mmq, gpu_quantize,
                            gpu_repack, oracle_q8, oracle_w, sample_rows, say, workload)
from tests.layout_ref import q8_image, q8_regions, repack_reference

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")

LARGE, SMALL, SKINNY = mmq.MMQ_TILE_LARGE, mmq.MMQ_TILE_SMALL, mmq.MMQ_TILE_SKINNY
MEDIUM, HALF = mmq.MMQ_TILE_MEDIUM, mmq.MMQ_TILE_HALF
CONFIGS = ["tiny", "qproj", "gateup", "down"]
SWEEP = [f"sweep_m{m}" for m in synth.SWEEP_M]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- quantize
def check_q8(got: np.ndarray, x: np.ndarray) -> None:
    """The q8 buffer of x, in two checks: (i) q, the f16 bits of da and sa bit-exact against
    the oracle's quantization; (ii) the GEMM's derived planes against the layout reference
    built from those same oracle fields."""
    M, K = x.shape
    q = oracle.quantize_q8_1(x)
    reg = q8_regions(got, M, K)
    assert np.array_equal(reg["qs"], q.qs), f"{np.count_nonzero(reg['qs'] != q.qs)} q differ"
    da_bits = (reg["words"] & 0xFFFF).astype(np.uint16)
    sa = (reg["words"] >> 16).astype(np.uint16).view(np.int16).astype(np.int32)
    assert np.array_equal(da_bits, q.da_bits), "da differs"
    assert np.array_equal(sa, q.sa), "sa differs"
    want = q8_image(q)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} plane bytes differ"


@pytest.mark.parametrize("name", CONFIGS + SWEEP)
def test_quantize_bitexact(name):
    W = workload(name)
    say("quantize", name, W["x"].shape)
    check_q8(gpu_quantize(W["x"]).cpu().numpy(), W["x"])


def test_quantize_edge_blocks(golden_dir):
    with open(os.path.join(golden_dir, "q8_1_worked_blocks.json")) as f:
        blocks = json.load(f)["blocks"]
    x = np.stack([np.array([int(h, 16) for h in b["x_f32_bits"]], np.uint32).view(np.float32)
                  for b in blocks])
    for shape in [(len(blocks), 32), (1, 32 * len(blocks))]:
        xs = x.reshape(shape)
        say("quantize edge blocks", shape)
        check_q8(gpu_quantize(xs).cpu().numpy(), xs)


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (37, 256), (129, 4128)])
def test_quantize_ragged(M, K):
    x = synth.activations("normal_outliers", M, K, M * 31 + K)
    say("quantize ragged", M, K)
    check_q8(gpu_quantize(x).cpu().numpy(), x)


# ----------------------------------------------------------------------------- repack
@pytest.mark.parametrize("name", ["tiny", "qproj", "gateup", "down"])
def test_repack_bytes(name):
    W = workload(name)
    say("repack", name, W["N"], W["K"])
    got = gpu_repack(W["w"], W["N"], W["K"]).cpu().numpy()
    assert np.array_equal(got, repack_reference(W["w"]))


@pytest.mark.parametrize("N,K", [(1, 256), (33, 512), (95, 768)])
def test_repack_ragged_rows(N, K):
    f = synth.q4k_random_fields(N, K, N + K)
    w = synth.q4k_pack(f)
    say("repack ragged", N, K)
    got = gpu_repack(w, N, K).cpu().numpy()
    assert np.array_equal(got, repack_reference(w))


# ----------------------------------------------------------------------------- block dots
@pytest.mark.parametrize("tile", [LARGE, HALF, MEDIUM, SMALL])
def test_blockdots_tiny_every_element(tile):
    W = workload("tiny")
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    say("blockdots tiny full", tile)
    S = gpu_blockdots(M, N, K, q8, rep, 0, M, 0, N, force_tile=tile)
    want = oracle.block_dots(oracle_q8("tiny"), oracle_w("tiny"), range(M), range(N))
    assert np.array_equal(S.astype(np.int64), want)


WINDOWS = {  # (i0, i1, j0, j1) -- corners, tile edges and ragged tails
    "qproj": [(0, 40, 0, 70), (120, 136, 4064, 4096), (2016, 2048, 1000, 1040)],
    "gateup": [(0, 33, 10976, 11008), (1900, 1950, 5000, 5030)],
    "down": [(2000, 2048, 0, 64), (500, 530, 4000, 4096)],
}


@pytest.mark.parametrize("name", sorted(WINDOWS))
@pytest.mark.parametrize("tile", [LARGE, HALF, SMALL])
def test_blockdots_windows(name, tile):
    W = workload(name)
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    for (i0, i1, j0, j1) in WINDOWS[name]:
        say("blockdots", name, tile, (i0, i1, j0, j1))
        S = gpu_blockdots(M, N, K, q8, rep, i0, i1, j0, j1, force_tile=tile)
        want = oracle.block_dots(oracle_q8(name), oracle_w(name), range(i0, i1), range(j0, j1))
        assert np.array_equal(S.astype(np.int64), want)


# ----------------------------------------------------------------------------- the product
@pytest.mark.parametrize("tile", [LARGE, HALF, MEDIUM, SMALL])
def test_mmq_tiny_every_element(tile):
    W = workload("tiny")
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    say("mmq tiny", tile)
    C = gpu_mmq(M, N, K, q8, rep, force_tile=tile)
    C_ref = oracle.mmq(oracle_q8("tiny"), oracle_w("tiny"))
    _, T = oracle.mmq_terms(oracle_q8("tiny"), oracle_w("tiny"))
    r = assert_within_tolerance(C, C_ref, T)
    say("max |err|/T", r)


def test_mmq_qproj_every_element():
    """The 2048 x 4096 x 4096 product in the launch configuration the benchmark times."""
    name = "qproj"
    W = workload(name)
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    say("mmq qproj full")
    C = gpu_mmq(M, N, K, q8, rep)
    assert mmq.mmq_last_kernel()["tile"] == LARGE
    C_terms, T = oracle.mmq_terms(oracle_q8(name), oracle_w(name))
    C_ref = oracle.mmq(oracle_q8(name), oracle_w(name))
    assert np.all(np.abs(C_ref - C_terms) <= 1e-12 * T)
    r = assert_within_tolerance(C, C_ref, T)
    say("max |err|/T", r)


@pytest.mark.parametrize("name", ["gateup", "down"] + [n for n in SWEEP if n != "sweep_m8192"])
def test_mmq_every_element(name):
    """Every element of the full-size products, in the launch the guard chooses."""
    W = workload(name)
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    say("mmq every element", name, (M, N, K))
    C = gpu_mmq(M, N, K, q8, rep)
    C_ref = oracle.mmq(oracle_q8(name), oracle_w(name))
    _, T = oracle.mmq_terms(oracle_q8(name), oracle_w(name))
    r = assert_within_tolerance(C, C_ref, T)
    say("max |err|/T", r, "tile", mmq.mmq_last_kernel()["tile"])


@pytest.mark.parametrize("name", ["sweep_m8192"])
def test_mmq_sampled_rows(name):
    W = workload(name)
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    say("mmq", name, (M, N, K))
    C = gpu_mmq(M, N, K, q8, rep)
    rows = sample_rows(M)
    C_ref = oracle.mmq(oracle_q8(name), oracle_w(name), rows=rows)
    _, T = oracle.mmq_terms(oracle_q8(name), oracle_w(name), rows=rows)
    r = assert_within_tolerance(C[rows], C_ref, T)
    say("max |err|/T", r, "rows", len(rows))


@pytest.mark.parametrize("name", synth.SHARE8)
def test_mmq_per_gpu_share_shapes(name):
    """One GPU's share of an 8-way column split (N = 512 or 1376), under the guard's tile and
    the large tile, on sampled rows."""
    W = workload(name)
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    rows = sample_rows(M)
    C_ref = oracle.mmq(oracle_q8(name), oracle_w(name), rows=rows)
    _, T = oracle.mmq_terms(oracle_q8(name), oracle_w(name), rows=rows)
    for tile in (0, LARGE):
        say("mmq share", name, (M, N, K), "tile", tile)
        C = gpu_mmq(M, N, K, q8, rep, force_tile=tile)
        r = assert_within_tolerance(C[rows], C_ref, T)
        say("max |err|/T", r)


@pytest.mark.parametrize("name", ["tiny", "sweep_m1", "sweep_m16", "sweep_m128"])
def test_mmq_skinny_every_element(name):
    """The skinny kernel (K split over the wavefronts of a workgroup) on every element."""
    W = workload(name)
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    say("mmq skinny", name, (M, N, K))
    C = gpu_mmq(M, N, K, q8, rep, force_tile=SKINNY)
    assert mmq.mmq_last_kernel()["tile"] == SKINNY
    C_ref = oracle.mmq(oracle_q8(name), oracle_w(name))
    _, T = oracle.mmq_terms(oracle_q8(name), oracle_w(name))
    r = assert_within_tolerance(C, C_ref, T)
    say("max |err|/T", r)


@pytest.mark.parametrize("M,N,K,lazy", [(200, 4096, 4096, True), (256, 1376, 4096, True),
                                        (33, 4096, 11008, False)])
def test_mmq_guard_skinny_range_every_element(M, N, K, lazy):
    """Shapes the guard gives to the skinny kernel, every element: ragged token tiles in the
    two-workgroups-per-CU form (grid above the compute units; token operands loaded two
    blocks ahead), and 5 to 6 super-blocks per wavefront in the one-round form (the next
    super-block's loads in flight)."""
    x = synth.activations("normal_outliers", M, K, 7000 + M)
    w, _ = synth.q4k_weights("fit", N, K, 7001 + M)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, N, K)
    say("mmq guard skinny", (M, N, K))
    C = gpu_mmq(M, N, K, q8, rep)
    info = mmq.mmq_last_kernel()
    assert info["tile"] == SKINNY and (info["grid"] > 256) == lazy
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    r = assert_within_tolerance(C, oracle.mmq(q, wo), T)
    say("max |err|/T", r)


def test_mmq_skinny_deterministic():
    x = synth.activations("normal_outliers", 40, 2816, 15)
    w, f = synth.q4k_weights("fit", 70, 2816, 16)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, 70, 2816)
    say("mmq skinny deterministic")
    a = gpu_mmq(40, 70, 2816, q8, rep, force_tile=SKINNY)
    b = gpu_mmq(40, 70, 2816, q8, rep, force_tile=SKINNY)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    assert_within_tolerance(a, oracle.mmq(q, wo), T)


def test_mmq_tiles_agree_bitwise_and_deterministic():
    """The template's four instantiations add the same terms in the same order: identical
    bits, on ragged M and N."""
    x = synth.activations("normal_outliers", 300, 1024, 5)
    w, f = synth.q4k_weights("fit", 200, 1024, 6)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, 200, 1024)
    say("mmq tiles agree")
    a = gpu_mmq(300, 200, 1024, q8, rep, force_tile=LARGE)
    for tile in (SMALL, MEDIUM, HALF, LARGE):
        b = gpu_mmq(300, 200, 1024, q8, rep, force_tile=tile)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), tile


def test_mmq_lds_fallback_reported():
    x = synth.activations("normal", 96, 512, 1)
    w, f = synth.q4k_weights("random_fields", 64, 512, 2)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, 64, 512)
    large_lds = mmq.mmq_plan(96, 64, 512, 1 << 20, force_tile=LARGE)["lds_bytes"]
    say("mmq lds fallback")
    C = gpu_mmq(96, 64, 512, q8, rep, lds_budget=large_lds - 1)
    info = mmq.mmq_last_kernel()
    assert info["tile"] == SMALL and info["fallback"] == 1
    assert info["reason"] == mmq.MMQ_REASON_LDS_FALLBACK
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    assert_within_tolerance(C, oracle.mmq(q, wo), T)
    with pytest.raises(mmq.MMQError) as e:
        gpu_mmq(96, 64, 512, q8, rep, lds_budget=1024)
    assert e.value.status == mmq.MMQ_E_LDS


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (33, 33, 256), (1, 1, 256), (130, 97, 512),
                                   (64, 4097, 256), (257, 40, 1280)])
def test_mmq_edge_shapes(M, N, K):
    x = synth.activations("normal_outliers", M, K, M + N + K)
    w, f = synth.q4k_weights("random_fields", N, K, M * N + K)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, N, K)
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    C_ref = oracle.mmq(q, wo)
    for tile in (LARGE, HALF, SMALL, SKINNY):
        say("mmq edge", (M, N, K), tile)
        C = gpu_mmq(M, N, K, q8, rep, force_tile=tile)
        assert_within_tolerance(C, C_ref, T)


def test_mmq_integer_case_exact():
    """d = 1, sc = 1, dmin = 0, integer activations with a +-127 per block: C = x @ v^T exactly."""
    rng = np.random.default_rng(3)
    M, N, K = 160, 96, 1024
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 7] = rng.choice([-127.0, 127.0], (M, K // 32))
    f = {"d_bits": np.full((N, K // 256), 0x3C00, np.uint16),
         "dmin_bits": np.zeros((N, K // 256), np.uint16),
         "sc": np.ones((N, K // 32), np.uint8),
         "m": rng.integers(0, 64, (N, K // 32), dtype=np.uint8),
         "v": rng.integers(0, 16, (N, K), dtype=np.uint8)}
    w = synth.q4k_pack(f)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, N, K)
    want = (x.astype(np.int64) @ f["v"].astype(np.int64).T).astype(np.float64)
    for tile in (LARGE, HALF, SMALL):
        say("mmq integer case", tile)
        C = gpu_mmq(M, N, K, q8, rep, force_tile=tile)
        assert np.array_equal(C.astype(np.float64), want)


def test_mmq_degenerate_inputs():
    """All-zero activations give exactly 0; zero sc or zero m removes one term."""
    M, N, K = 70, 64, 512
    w, f = synth.q4k_weights("random_fields", N, K, 9)
    rep = gpu_repack(w, N, K)
    say("mmq zero activations")
    C = gpu_mmq(M, N, K, gpu_quantize(np.zeros((M, K), np.float32)), rep)
    assert np.all(C == 0.0)
    x = synth.activations("normal", M, K, 10)
    q8 = gpu_quantize(x)
    q = oracle.quantize_q8_1(x)
    for which in ("sc", "m"):
        f2 = dict(f, **{which: np.zeros_like(f[which])})
        w2 = synth.q4k_pack(f2)
        say("mmq zero", which)
        C = gpu_mmq(M, N, K, q8, gpu_repack(w2, N, K))
        wo = oracle.decode_q4_K(w2)
        _, T = oracle.mmq_terms(q, wo)
        assert_within_tolerance(C, oracle.mmq(q, wo), T)
