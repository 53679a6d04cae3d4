"""The quantize-fused product for few tokens, mmq_q4K_f32, through the C ABI (needs a GPU).

Bars:
- C bit for bit equal to quantize_q8_1 followed by mmq_q4K_q8_1_ex with the kernel the fused
  call uses: the decode tile's vector-ALU form for M <= 8 (taken under an LDS budget below
  the matrix-unit form's), the skinny tile above (each fused kernel quantizes with the
  prepass's arithmetic and then does its unfused twin's arithmetic in the same order);
- within 1e-5 * T of the oracle, as for the unfused product.
Shapes cover one and several token tiles, ragged M and N, K of one super-block (most
wavefronts of a workgroup get no super-block) and K with super-blocks that do not divide
evenly over the wavefronts.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_within_tolerance, gpu_repack, say, to_dev

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()


def fused_tile(M):
    return mmq.MMQ_TILE_GEMV if M <= 8 else mmq.MMQ_TILE_SKINNY


def valu_form_budget(M, N, K):
    """An LDS budget that leaves M <= 8 tokens to the decode tile's vector-ALU form, the
    unfused twin of the fused kernel: one byte below the matrix-unit form's LDS where the guard
    takes that form (its LDS depends on the wavefront count N calls for), else no budget."""
    p = mmq.mmq_plan(M, N, K, 160 * 1024, force_tile=mmq.MMQ_TILE_GEMV)
    return p["lds_bytes"] - 1 if p["block_m"] == 16 else 0


def two_step(x_dev, M, N, K, rep):
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")
    mmq.quantize_q8_1(x_dev, M, K, q8)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_q8_1_ex(M, N, K, q8, rep, C, force_tile=fused_tile(M),
                        lds_budget=valu_form_budget(M, N, K) if M <= 8 else 0)
    torch.cuda.synchronize()
    if M <= 8:
        assert mmq.mmq_last_kernel()["block_m"] <= 8, "the two-step path must take the vector-ALU form"
    return C.cpu().numpy()


def fused(x_dev, M, N, K, rep):
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_f32(M, N, K, x_dev, rep, C)
    torch.cuda.synchronize()
    return C.cpu().numpy()


SHAPES = [(1, 4096, 4096), (2, 256, 512), (7, 33, 768), (16, 4096, 4096), (32, 512, 1024),
          (33, 96, 2048), (100, 65, 2304), (128, 4096, 4096), (5, 40, 256), (3, 64, 11008),
          (8, 4097, 4096), (9, 70, 1024), (4, 16, 9472), (1, 1, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fused_equals_prepass_then_unfused(M, N, K):
    x = synth.activations("normal_outliers", M, K, 9000 + M + K)
    w, _ = synth.q4k_weights("fit", N, K, 9001 + N)
    rep = gpu_repack(w, N, K)
    x_dev = to_dev(x)
    say("fused vs two-step", M, N, K)
    want = two_step(x_dev, M, N, K, rep)
    got = fused(x_dev, M, N, K, rep)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{np.count_nonzero(got.view(np.uint32) != want.view(np.uint32))} elements differ"
    info = mmq.mmq_last_kernel()
    assert info["tile"] == fused_tile(M) and info["reason"] == mmq.MMQ_REASON_FUSED


@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (9, 70, 1024), (40, 33, 768),
                                   (1, 4096, 4096), (8, 4096, 4096), (128, 4096, 4096)])
def test_fused_against_the_oracle(M, N, K):
    x = synth.activations("normal_outliers", M, K, 9100 + M)
    w, _ = synth.q4k_weights("random_fields", N, K, 9101 + N)
    rep = gpu_repack(w, N, K)
    say("fused vs oracle", M, N, K)
    got = fused(to_dev(x), M, N, K, rep)
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    r = assert_within_tolerance(got, oracle.mmq(q, wo), T)
    say("max |err|/T", r)


def test_fused_edge_blocks(golden_dir):
    """The worked q8_1 blocks (zero block, scale that underflows, reciprocal that overflows)
    as activations: the in-kernel quantization must match the prepass's bytes exactly."""
    with open(os.path.join(golden_dir, "q8_1_worked_blocks.json")) as f:
        blocks = json.load(f)["blocks"]
    x8 = np.stack([np.array([int(h, 16) for h in b["x_f32_bits"]], np.uint32).view(np.float32)
                   for b in blocks]).reshape(1, -1)              # one super-block of 8 blocks
    assert x8.shape == (1, 256)
    x = np.concatenate([x8, x8[:, ::-1], -x8], axis=0)          # 3 tokens
    M, K, N = 3, 256, 64
    w, _ = synth.q4k_weights("random_fields", N, K, 9200)
    rep = gpu_repack(w, N, K)
    x_dev = to_dev(np.ascontiguousarray(x))
    say("fused edge blocks")
    want = two_step(x_dev, M, N, K, rep)
    got = fused(x_dev, M, N, K, rep)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_fused_repeated_calls_and_streams():
    """Back-to-back calls on a side stream into distinct outputs agree with one another."""
    M, N, K = 4, 512, 2048
    x = synth.activations("normal", M, K, 9300)
    w, _ = synth.q4k_weights("fit", N, K, 9301)
    rep = gpu_repack(w, N, K)
    x_dev = to_dev(x)
    ref = fused(x_dev, M, N, K, rep)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = [torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") for _ in range(4)]
    say("fused on a side stream")
    for C in outs:
        mmq.mmq_q4K_f32(M, N, K, x_dev, rep, C, stream=s)
    s.synchronize()
    for C in outs:
        assert np.array_equal(C.cpu().numpy(), ref)
