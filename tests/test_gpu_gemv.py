"""The decode tile for a handful of tokens (MMQ_TILE_GEMV) against the CPU oracle.

Bar: f32 outputs within 1e-5 * T per element (T from the oracle, float64), every element;
results deterministic. The tile is the guard's choice for M <= 16, in two forms: vector-ALU
dot products (up to M = 4, and up to M = 8 when the rows need more than one round of
workgroups) and a 16 x 16 int8 MFMA per block (from M = 9, and from M = 5 within one round),
so the token sweep's M = 1 and M = 16 shapes run through it by default.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (assert_within_tolerance, gpu_mmq, gpu_quantize, gpu_repack,
                            oracle_q8, oracle_w, say, workload)

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")

GEMV = mmq.MMQ_TILE_GEMV


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()


def _check(M, N, K, seed, kind="normal_outliers", wkind="random_fields", force=GEMV,
           lds_budget=0):
    x = synth.activations(kind, M, K, seed)
    w, _ = synth.q4k_weights(wkind, N, K, seed + 1)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, N, K)
    say("gemv", (M, N, K), "seed", seed, "lds budget", lds_budget)
    C = gpu_mmq(M, N, K, q8, rep, force_tile=force, lds_budget=lds_budget)
    info = mmq.mmq_last_kernel()
    assert info["tile"] == GEMV
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    r = assert_within_tolerance(C, oracle.mmq(q, wo), T)
    say("max |err|/T", r)
    return C, info


@pytest.mark.parametrize("name", ["sweep_m1", "sweep_m16"])
def test_gemv_decode_shapes_every_element(name):
    """The token sweep's decode shapes, M = 1 and M = 16, by the guard's own choice."""
    W = workload(name)
    M, N, K = W["M"], W["N"], W["K"]
    q8 = gpu_quantize(W["x"])
    rep = gpu_repack(W["w"], N, K)
    say("gemv", name, (M, N, K))
    C = gpu_mmq(M, N, K, q8, rep, force_tile=0)
    info = mmq.mmq_last_kernel()
    assert info["tile"] == GEMV
    assert info["reason"] == mmq.MMQ_REASON_DECODE
    _, T = oracle.mmq_terms(oracle_q8(name), oracle_w(name))
    r = assert_within_tolerance(C, oracle.mmq(oracle_q8(name), oracle_w(name)), T)
    say("max |err|/T", r)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8, 9, 12, 13, 16])
def test_gemv_every_token_count(M):
    """Groups of 1, 2, 4 and 8 tokens, and a partly filled last group (M = 3, 5, 7, 9, 12, 13)."""
    C, info = _check(M, 160, 1024, 100 + M)
    assert info["block_m"] == mmq.mmq_plan(M, 160, 1024, 160 * 1024, force_tile=GEMV)["block_m"]
    assert info["block_m"] >= min(M, 4)


# LDS of the matrix-unit form; one byte less leaves 5-8 tokens to the vector-ALU form
MFMA_FORM_LDS = mmq.mmq_plan(8, 160, 1024, 160 * 1024, force_tile=GEMV)["lds_bytes"]


@pytest.mark.parametrize("M,N,K", [(5, 160, 1024), (6, 96, 2816), (7, 4097, 256),
                                   (8, 70, 11008)])
def test_gemv_both_forms_from_5_to_8_tokens(M, N, K):
    """5 to 8 tokens run in either form, by the guard's choice of form: the matrix-unit form
    when its grid runs in one round and fits the LDS, else the vector-ALU form."""
    a, ia = _check(M, N, K, 300 + M)
    b, ib = _check(M, N, K, 300 + M, lds_budget=MFMA_FORM_LDS - 1)
    assert ib["threads"] == 512 and ib["block_m"] == 8
    assert ia["threads"] == (1024 if (N + 15) // 16 <= 256 else 512)


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 256),        # one row, one super-block (15 of 16 slices idle)
    (3, 33, 256),       # three row blocks, the last with one real row
    (2, 96, 512),       # the second half of a tile
    (4, 4097, 256),     # 257 row blocks
    (1, 64, 9472),      # 37 super-blocks: 2 or 3 per slice, the last step partly idle
    (5, 70, 11008),     # 43 super-blocks over 16 slices, a ragged token group
    (16, 200, 2816),    # 11 super-blocks: 5 slices idle, wavefront 3 without a step
])
def test_gemv_edge_shapes(M, N, K):
    _check(M, N, K, M * 1000 + N + K)


def test_gemv_extreme_values():
    """Weights with the largest nibbles and scales, activations with outliers per block."""
    _check(4, 96, 1024, 7, kind="normal_outliers", wkind="fit")
    _check(3, 64, 768, 8, kind="normal_outliers", wkind="random_fields")


def test_gemv_integer_case_exact():
    """d = 1, sc = 1, dmin = 0, integer activations with a +-127 per block: C = x @ v^T."""
    rng = np.random.default_rng(11)
    M, N, K = 13, 96, 1024
    x = rng.integers(-127, 128, (M, K)).astype(np.float32)
    x.reshape(M, K // 32, 32)[:, :, 5] = rng.choice([-127.0, 127.0], (M, K // 32))
    f = {"d_bits": np.full((N, K // 256), 0x3C00, np.uint16),
         "dmin_bits": np.zeros((N, K // 256), np.uint16),
         "sc": np.ones((N, K // 32), np.uint8),
         "m": rng.integers(0, 64, (N, K // 32), dtype=np.uint8),
         "v": rng.integers(0, 16, (N, K), dtype=np.uint8)}
    w = synth.q4k_pack(f)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, N, K)
    say("gemv integer case")
    C = gpu_mmq(M, N, K, q8, rep, force_tile=GEMV)
    want = x.astype(np.int64) @ f["v"].astype(np.int64).T
    assert np.array_equal(C.astype(np.int64), want)


def test_gemv_deterministic_and_agrees_with_skinny():
    x = synth.activations("normal_outliers", 9, 2816, 21)
    w, _ = synth.q4k_weights("fit", 70, 2816, 22)
    q8 = gpu_quantize(x)
    rep = gpu_repack(w, 70, 2816)
    say("gemv deterministic")
    a = gpu_mmq(9, 70, 2816, q8, rep, force_tile=GEMV)
    b = gpu_mmq(9, 70, 2816, q8, rep, force_tile=GEMV)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    s = gpu_mmq(9, 70, 2816, q8, rep, force_tile=mmq.MMQ_TILE_SKINNY)
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    assert_within_tolerance(a, s.astype(np.float64), 2 * T)
