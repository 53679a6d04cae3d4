"""The hot path under HIP graph capture (needs a GPU).

Every entry point launches its kernels on the caller's stream and allocates nothing, so a
whole step can be captured into a graph and replayed without the host's per-launch cost.
Each case captures a step, replays it several times with eager work and synchronizations
between the replays, and checks every replay bit for bit against the eager result of the
same entry points (the kernels are deterministic).
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

mmq = pytest.importorskip("q4_q8_int8_amd")
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    yield
    torch.cuda.synchronize()


def _replay_and_check(g, out, want, disturb):
    for i in range(3):
        out.fill_(float("nan"))
        disturb()                      # eager work on the same buffers' stream in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, want), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("M,N,K", [(2048, 4096, 4096), (1, 4096, 4096), (12, 4096, 4096),
                                   (8, 11008, 1024), (6, 8192, 512), (16, 1024, 2048),
                                   (100, 512, 1024)])
def test_integer_step_in_a_graph(M, N, K):
    """The guard's choice under capture: the large tile, the decode tile's vector-ALU form
    and its matrix-unit form with 16, 4 and 8 wavefronts, and the small tile."""
    x = to_dev(synth.activations("normal_outliers", M, K, 7000 + M))
    w, _ = synth.q4k_weights("fit", N, K, 7001)
    rep = torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    mmq.repack_q4_K(to_dev(w), N, K, rep)
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("graph: integer step eager", M, N, K)
    mmq.quantize_q8_1(x, M, K, q8)
    mmq.mmq_q4K_q8_1(M, N, K, q8, rep, C)
    torch.cuda.synchronize()
    want = C.cpu().numpy()

    say("graph: capture", M, N, K)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mmq.quantize_q8_1(x, M, K, q8)
            mmq.mmq_q4K_q8_1(M, N, K, q8, rep, C)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def disturb():  # scribble over the q8 buffer eagerly; the replay must rewrite it
        q8.fill_(0x55)
    say("graph: replays", M, N, K)
    _replay_and_check(g, C, want, disturb)


@pytest.mark.parametrize("M,N,K,tile,split", [(768, 1376, 2048, "half", False),
                                               (200, 4096, 4096, "auto", False),
                                               (2048, 512, 4096, "auto", True)])
def test_ex_options_in_a_graph(M, N, K, tile, split):
    """The half tile, the skinny kernel's two-workgroups-per-CU form, and split-K (the GEMM
    writing its partial planes into the caller's workspace, then the second pass) captured
    with the quantize step."""
    x = to_dev(synth.activations("normal_outliers", M, K, 7100 + M))
    w, _ = synth.q4k_weights("fit", N, K, 7101)
    rep = torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    mmq.repack_q4_K(to_dev(w), N, K, rep)
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = None
    if split:
        ws = torch.empty(mmq.mmq_workspace_bytes(M, N, K) // 4, dtype=torch.float32,
                         device="cuda")
    force = mmq.MMQ_TILE_HALF if tile == "half" else mmq.MMQ_TILE_AUTO

    def step():
        mmq.quantize_q8_1(x, M, K, q8)
        mmq.mmq_q4K_q8_1_ex(M, N, K, q8, rep, C, force_tile=force, workspace=ws)

    say("graph: ex options eager", M, N, K, tile, split)
    step()
    torch.cuda.synchronize()
    want = C.cpu().numpy()
    info = mmq.mmq_last_kernel()
    if tile == "half":
        assert info["tile"] == mmq.MMQ_TILE_HALF
    if split:
        assert info["splits"] > 1
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def disturb():  # scribble over the q8 buffer and the workspace eagerly
        q8.fill_(0x55)
        if ws is not None:
            ws.fill_(float("nan"))
    say("graph: ex options replays", M, N, K)
    _replay_and_check(g, C, want, disturb)


def test_f16_path_in_a_graph():
    M, N, K = 512, 1024, 2048
    x = to_dev(synth.activations("normal_outliers", M, K, 7002))
    w, _ = synth.q4k_weights("fit", N, K, 7003)
    w_dev = to_dev(w)
    xa = torch.empty(M * K, dtype=torch.int16, device="cuda")
    wf = torch.empty(N * K, dtype=torch.int16, device="cuda")
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("graph: f16 path eager", M, N, K)
    mmq.convert_f32_f16(x, M, K, xa)
    mmq.dequantize_q4_K_f16(w_dev, N, K, wf)
    mmq.gemm_f16(M, N, K, xa, wf, C)
    torch.cuda.synchronize()
    want = C.cpu().numpy()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mmq.convert_f32_f16(x, M, K, xa)
            mmq.dequantize_q4_K_f16(w_dev, N, K, wf)
            mmq.gemm_f16(M, N, K, xa, wf, C)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def disturb():
        xa.fill_(0x3C00)
        wf.fill_(0)
    say("graph: f16 replays", M, N, K)
    _replay_and_check(g, C, want, disturb)


def test_side_stream_is_honoured():
    """Kernels run on the stream passed in: work on a side stream, ordered by events only."""
    M, N, K = 256, 512, 1024
    x = to_dev(synth.activations("normal", M, K, 7004))
    w, _ = synth.q4k_weights("fit", N, K, 7005)
    rep = torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    mmq.repack_q4_K(to_dev(w), N, K, rep)
    q8 = torch.zeros(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device="cuda")
    C0 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mmq.quantize_q8_1(x, M, K, q8)
    mmq.mmq_q4K_q8_1(M, N, K, q8, rep, C0)
    torch.cuda.synchronize()
    say("side stream")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    q8b = torch.zeros_like(q8)
    C1 = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    mmq.quantize_q8_1(x, M, K, q8b, stream=s)
    mmq.mmq_q4K_q8_1(M, N, K, q8b, rep, C1, stream=s)
    s.synchronize()
    assert np.array_equal(C1.cpu().numpy(), C0.cpu().numpy())


def test_fused_few_token_step_in_a_graph():
    M, N, K = 2, 4096, 4096
    x = to_dev(synth.activations("normal_outliers", M, K, 7006))
    w, _ = synth.q4k_weights("fit", N, K, 7007)
    rep = torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device="cuda")
    mmq.repack_q4_K(to_dev(w), N, K, rep)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("graph: fused step eager", M, N, K)
    mmq.mmq_q4K_f32(M, N, K, x, rep, C)
    torch.cuda.synchronize()
    want = C.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mmq.mmq_q4K_f32(M, N, K, x, rep, C)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def disturb():
        C.fill_(0.0)
    say("graph: fused replays", M, N, K)
    _replay_and_check(g, C, want, disturb)

