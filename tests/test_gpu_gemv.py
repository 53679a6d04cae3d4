"""The decode tile for a handful of tokens (MMQ_TILE_GEMV) against the CPU oracle.

Bar: f32 outputs within 1e-5 * T per element (T from the oracle, float64), every element;
results deterministic. The tile is the guard's choice for M <= 16, in two forms: vector-ALU
dot products (up to M = 4) and a 16 x 16 int8 MFMA per block (from M = 5) with 16, 8 or 4
wavefronts per workgroup by the number of 16-row blocks, so the token sweep's M = 1 and
M = 16 shapes run through it by default. The vector-ALU form still serves 5 to 8 tokens under
an LDS budget below the matrix-unit form's, and is tested that way too.
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


def mfma_waves(N):
    """The matrix-unit form's wavefronts per workgroup: its N / 16 workgroups fit the 256
    compute units that mmq_plan assumes once (16), twice (8) or not (4)."""
    nrb = (N + 15) // 16
    return 16 if nrb <= 256 else (8 if nrb <= 512 else 4)


def valu_budget(M, N, K):
    """One byte below the matrix-unit form's LDS: leaves 5-8 tokens to the vector-ALU form."""
    return mmq.mmq_plan(M, N, K, 160 * 1024, force_tile=GEMV)["lds_bytes"] - 1


@pytest.mark.parametrize("M,N,K", [(5, 160, 1024), (6, 96, 2816), (7, 4097, 256),
                                   (8, 70, 11008), (6, 8192, 512)])
def test_gemv_both_forms_from_5_to_8_tokens(M, N, K):
    """5 to 8 tokens run in either form: the matrix-unit form by the guard's choice, the
    vector-ALU form under an LDS budget one byte below it."""
    a, ia = _check(M, N, K, 300 + M)
    assert ia["block_m"] == 16 and ia["threads"] == 64 * mfma_waves(N)
    assert ia["block_n"] == (32 if mfma_waves(N) == 8 else 16)
    b, ib = _check(M, N, K, 300 + M, lds_budget=valu_budget(M, N, K))
    assert ib["threads"] == 512 and ib["block_m"] == 8


@pytest.mark.parametrize("M,N,K", [
    (16, 4112, 1024),   # 257 16-row blocks: 129 of 32 rows (the last with 16), 8 wavefronts
    (5, 4100, 2816),    # 8 wavefronts over 11 super-blocks: three take a second one
    (6, 8192, 4096),    # 256 blocks of 32 rows: 8 wavefronts, two super-blocks each
    (7, 4104, 512),     # 129 blocks of 32 rows, the last with 8 rows: a half with none
    (9, 8208, 9472),    # 513 row blocks: 4 wavefronts over 37 super-blocks (10, 9, 9, 9)
    (16, 11008, 4096),  # the gate/up rows: 4 wavefronts, four super-blocks each
])
def test_gemv_matrix_form_wave_counts(M, N, K):
    """The matrix-unit form with 8 wavefronts and 32 rows and with 4 wavefronts and 16 rows per
    workgroup, each wavefront taking one or several super-blocks (the next one's weights
    loaded during this one), every element."""
    C, info = _check(M, N, K, 700 + M)
    assert info["block_m"] == 16 and info["threads"] == 64 * mfma_waves(N)
    assert info["block_n"] == (32 if mfma_waves(N) == 8 else 16)


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 256),        # one row, one super-block (15 of 16 slices idle)
    (3, 33, 256),       # three row blocks, the last with one real row
    (2, 96, 512),       # the second half of a tile
    (4, 4097, 256),     # 257 row blocks
    (1, 64, 9472),      # 37 super-blocks: 2 or 3 per slice, the last step partly idle
    (5, 70, 11008),     # 43 super-blocks over 16 slices, a ragged token group
    (16, 200, 2816),    # 11 super-blocks: 5 slices idle, wavefront 3 without a step
    (6, 1, 256),        # matrix-unit form: one row, one super-block, 15 wavefronts idle
    (12, 33, 512),      # three row blocks, the last with one real row, 4 tokens past M
])
@pytest.mark.parametrize("form", ["guard", "vector_alu"])
def test_gemv_edge_shapes(M, N, K, form):
    """By the guard's choice of form, and from 5 to 8 tokens also in the vector-ALU form."""
    if form == "vector_alu" and not 5 <= M <= 8:
        pytest.skip("the guard's form is the vector-ALU one below 5 tokens, the only one above 8")
    _check(M, N, K, M * 1000 + N + K, lds_budget=valu_budget(M, N, K) if form != "guard" else 0)


@pytest.mark.parametrize("M", [4, 3, 6])
def test_gemv_extreme_values(M):
    """Weights with the largest nibbles and scales, activations with outliers per block; 3 and
    4 tokens in the vector-ALU form, 6 in the matrix-unit form."""
    for (N, K, seed, wkind) in [(96, 1024, 7, "fit"), (64, 768, 8, "random_fields")]:
        _check(M, N, K, seed, kind="normal_outliers", wkind=wkind)


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
