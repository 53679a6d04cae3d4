"""mmq_q4K_q8_1_static, the entry point that allocates nothing (needs a GPU).

It runs mmq_q4K_q8_1_ex's kernels with the split-K workspace in the library's own 32 MiB
device array. Checked through the C ABI against mmq_q4K_q8_1_ex given a caller workspace of
the same size (so the guard makes the same plan): two calls in a row, the second with a
smaller product, bit for bit equal, and within the oracle's tolerance; the same call inside a
captured HIP graph, replayed; the refusals.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_within_tolerance, gpu_quantize, gpu_repack, say

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")

SCRATCH = 32 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()


def inputs(M, N, K, seed):
    x = synth.activations("normal_outliers", M, K, seed)
    w, _ = synth.q4k_weights("fit", N, K, seed + 1)
    return x, w, gpu_quantize(x), gpu_repack(w, N, K)


def both(M, N, K, q8, rep):
    ws = torch.empty(SCRATCH // 4, dtype=torch.float32, device="cuda")
    C_ex = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_q8_1_ex(M, N, K, q8, rep, C_ex, workspace=ws)
    torch.cuda.synchronize()
    plan_ex = mmq.mmq_last_kernel()
    C_st = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    mmq.mmq_q4K_q8_1_static(M, N, K, q8, rep, C_st)
    torch.cuda.synchronize()
    plan_st = mmq.mmq_last_kernel()
    return C_ex.cpu().numpy(), C_st.cpu().numpy(), plan_ex, plan_st


def test_static_scratch_matches_the_caller_workspace_twice():
    first = (128, 4096, 11008)    # split 4 ways: 8 MiB of partial planes
    second = (32, 1376, 2048)     # smaller, split 8 ways, over what the first call left
    for (M, N, K), seed in ((first, 9100), (second, 9200)):
        x, w, q8, rep = inputs(M, N, K, seed)
        say("static scratch", (M, N, K))
        C_ex, C_st, p_ex, p_st = both(M, N, K, q8, rep)
        assert p_st["splits"] > 1, "the call should take the split-K path"
        assert (p_st["tile"], p_st["splits"]) == (p_ex["tile"], p_ex["splits"])
        assert np.array_equal(C_st.view(np.uint32), C_ex.view(np.uint32))
        q = oracle.quantize_q8_1(x)
        wo = oracle.decode_q4_K(w)
        _, T = oracle.mmq_terms(q, wo)
        r = assert_within_tolerance(C_st, oracle.mmq(q, wo), T)
        say("splits", p_st["splits"], "max |err|/T", r)


def test_static_scratch_in_a_graph():
    M, N, K = 128, 4096, 11008
    x, w, q8, rep = inputs(M, N, K, 9300)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("static scratch eager")
    mmq.mmq_q4K_q8_1_static(M, N, K, q8, rep, C)
    torch.cuda.synchronize()
    want = C.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mmq.mmq_q4K_q8_1_static(M, N, K, q8, rep, C)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(3):
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        say("static scratch replay", i)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_static_scratch_refusals():
    M, N, K = 256, 16384, 1024           # 4 splits of 256 x 16384 floats: 64 MiB > 32 MiB
    x, w, q8, rep = inputs(M, N, K, 9400)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    with pytest.raises(mmq.MMQError) as e:
        mmq.mmq_q4K_q8_1_static(M, N, K, q8, rep, C, force_tile=mmq.MMQ_TILE_MEDIUM, splits=4)
    assert e.value.status == mmq.MMQ_E_ARG and "32 MiB" in str(e.value)
    # the guard plans within the scratch by itself
    say("static scratch: guard within 32 MiB")
    mmq.mmq_q4K_q8_1_static(M, N, K, q8, rep, C)
    torch.cuda.synchronize()
    assert mmq.mmq_last_kernel()["workspace_bytes"] <= SCRATCH
