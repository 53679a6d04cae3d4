"""Split-K through a caller's workspace (needs a GPU).

With a workspace the guard may split K over workgroups (on the tile its cost model prefers)
when the large tile's grid would leave compute units idle: each workgroup writes the partial sums of its
super-block range to a plane of the workspace and a second kernel adds the planes in split
order. Checked here: every element against the oracle at the shapes the guard splits (few
tokens, one GPU's share of a column split, ragged edges), forced split counts on every tile
of the template, bit-identical repeats, and the guard's choices and refusals.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_within_tolerance, gpu_quantize, gpu_repack, say

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")

MEDIUM, LARGE, SMALL = mmq.MMQ_TILE_MEDIUM, mmq.MMQ_TILE_LARGE, mmq.MMQ_TILE_SMALL
HALF = mmq.MMQ_TILE_HALF


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()


def case(M, N, K, seed, kind="fit"):
    x = synth.activations("normal_outliers", M, K, seed)
    w, _ = synth.q4k_weights(kind, N, K, seed + 1)
    q = oracle.quantize_q8_1(x)
    wo = oracle.decode_q4_K(w)
    _, T = oracle.mmq_terms(q, wo)
    return gpu_quantize(x), gpu_repack(w, N, K), oracle.mmq(q, wo), T


def run(M, N, K, q8, rep, ws_bytes, **kw):
    ws = torch.empty(max(ws_bytes, 16) // 4, dtype=torch.float32, device="cuda")
    ws.fill_(float("nan"))                     # stale contents must not matter
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_q8_1_ex(M, N, K, q8, rep, C, workspace=ws if ws_bytes else None, **kw)
    torch.cuda.synchronize()
    return C.cpu().numpy(), mmq.mmq_last_kernel()


@pytest.mark.parametrize("M,N,K", [(128, 4096, 11008), (2048, 512, 4096), (32, 1376, 2048),
                                   (100, 700, 2816), (256, 1024, 1024)])
def test_guard_splits_every_element(M, N, K):
    q8, rep, C_ref, T = case(M, N, K, M + N + K)
    need = mmq.mmq_workspace_bytes(M, N, K)
    say("split-K guard", (M, N, K), "workspace", need)
    C, info = run(M, N, K, q8, rep, need)
    assert info["tile"] in (MEDIUM, LARGE, SMALL, HALF) and info["reason"] == mmq.MMQ_REASON_SPLIT_K
    assert info["splits"] > 1 and info["workspace_bytes"] == need
    assert info["workspace_bytes"] == info["splits"] * M * N * 4
    r = assert_within_tolerance(C, C_ref, T)
    say("splits", info["splits"], "max |err|/T", r)


@pytest.mark.parametrize("tile,splits", [(MEDIUM, 2), (MEDIUM, 3), (MEDIUM, 11), (LARGE, 4),
                                         (SMALL, 5), (MEDIUM, 1), (HALF, 3)])
def test_forced_splits_every_element(tile, splits):
    M, N, K = 150, 300, 2816            # 11 super-blocks, ragged M and N
    q8, rep, C_ref, T = case(M, N, K, 31)
    say("split-K forced", tile, splits)
    C, info = run(M, N, K, q8, rep, splits * M * N * 4, force_tile=tile, splits=splits)
    assert info["tile"] == tile and info["splits"] == splits
    assert_within_tolerance(C, C_ref, T)


def test_split_results_repeat_bit_for_bit():
    M, N, K = 128, 4096, 11008
    q8, rep, _, _ = case(M, N, K, 77)
    need = mmq.mmq_workspace_bytes(M, N, K)
    say("split-K repeat")
    a, _ = run(M, N, K, q8, rep, need)
    b, _ = run(M, N, K, q8, rep, need)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_small_workspace_means_fewer_splits():
    M, N, K = 2048, 512, 11008
    q8, rep, C_ref, T = case(M, N, K, 78)
    full = mmq.mmq_workspace_bytes(M, N, K)
    say("split-K half workspace")
    C, info = run(M, N, K, q8, rep, full // 2)
    assert info["splits"] > 1 and info["workspace_bytes"] <= full // 2
    assert_within_tolerance(C, C_ref, T)
    say("split-K no room: no split")
    C, info = run(M, N, K, q8, rep, M * N * 4)    # one plane: too small for two splits
    assert info["splits"] == 1
    assert_within_tolerance(C, C_ref, T)


def test_forced_split_needs_room():
    M, N, K = 64, 256, 1024
    q8, rep, _, _ = case(M, N, K, 79)
    with pytest.raises(mmq.MMQError) as e:
        run(M, N, K, q8, rep, 3 * M * N * 4, force_tile=MEDIUM, splits=4)
    assert e.value.status == mmq.MMQ_E_ARG
