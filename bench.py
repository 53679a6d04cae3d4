"""Benchmark of the q4_K x q8_1 MMQ hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rotate R] [--no-cpu-baseline]
                    [--no-f16] [--sweep] [--decode [--shape M,N,K]]

Defaults: W = 500 warmup steps, and at least 300 ms of warmup whatever W is (the device's
clocks settle after ~50 ms of this load; the first q-proj steps take up to 1.5x the
steady-state time), then K = 200 timed steps.

Workload: the LLaMA-7B q-proj prefill product, M=2048 tokens, K=4096, N=4096, with
synthetic seeded inputs (synth.py: activations N(0,1) with 0.1% outliers x20, q4_K fit of
N(0, 0.02) weights). The weights are repacked once before timing (an offline, per-weight
step); one timed step is the whole per-batch path: quantize_q8_1 of the f32 activations
followed by the GEMM, with every input already resident in device memory. R copies of the
activations, weights and outputs are rotated (R = 8: about 740 MB for the steps, 470 MB for
the GEMM alone) so that no launch finds another launch's data in the 256 MB last-level
cache, as in a prefill where every product has its own weights.

Prints one JSON line. value = M*N*K / (time per step) in TMAC/s (1 MAC = one int8
multiply-accumulate), the time per step being the host wall clock over the K timed steps
between synchronizations. The GEMM kernel's own average duration, from HIP events around K
back-to-back launches on the stream it runs on, gives the roofline entry against the dense
int8 MFMA peak; its HBM traffic comes from the committed rocprofv3 counter summary of the
same kernel source (null once the kernel has changed since the counters were taken).

The line also carries `comparator_f16`: the same workload through the f16 comparator path
(convert_f32_f16, dequantize_q4_K_f16, gemm_f16), each kernel timed the same way, and the
two whole paths: per call, and with the weights resident in f16. `--no-f16` skips it.
`decode_m1` adds the one-token product against the same weights' shape (1 x 4096 x 4096) as
`--decode` times it; `--no-decode` skips it.

`--sweep` prints one line per configuration and tile instead, and `--decode` one line per
few-token shape (vector-ALU tile, skinny tile, fused call); neither is the benchmark line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0          # MI355X dense int8 MFMA, tera-ops/s (1 MAC = 2 ops)
F16_PEAK_TFLOPS = 2500.0         # MI355X dense f16 MFMA
HBM_PEAK_GBS = 8000.0
# MI355X FP32 vector rate without packed-FP32 instructions, which this library never uses:
# 16 FMA lanes per SIMD per cycle, 256 CUs x 4 SIMDs at 2.4 GHz (the published 157.3 TFLOP/s
# counts two FMAs per lane per packed instruction).
FP32_VECTOR_TFLOPS = 78.6
# The same FMA, measured with chains of independent v_fma_f32 on an MI355X at two wavefronts
# per SIMD (the GEMM's occupancy): 33.9 T FMA/s.
FP32_FMA_TFLOPS_AT_GEMM_OCCUPANCY = 67.8
# The shader clock while the q-proj GEMM runs, from s_memtime against s_memrealtime (100 MHz)
# read per workgroup in an instrumented copy of the kernel: 1.92-2.02 GHz, 1.99 on average.
# 16 FMA lanes per SIMD per cycle at that clock: 65.2 TFLOP/s.
GEMM_CLOCK_GHZ = 1.99
RESCALE_FMA_PER_EB = 2           # the rescale's FMAs per element-block (32-block of one C value)
PAGES_QPROJ_TMACS = 15.19        # the pages' best q-proj MMQ kernel: 34.36 GMAC in 2.262 ms
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mmq_qproj_traffic.json")
KERNEL_SOURCES = ["q4_q8_int8_amd/csrc/mmq_gemm.hip", "q4_q8_int8_amd/csrc/mmq_device.h",
                  "q4_q8_int8_amd/csrc/mmq_internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def epilogue_ceiling(M: int, N: int, K: int, gemm_us: float) -> dict:
    """The rescale's floor: RESCALE_FMA_PER_EB FP32 FMAs per element-block (M*N*K/32 of
    them) at the FP32 vector rate (non-packed, as built), the GEMM rate that floor allows as
    a fraction of the int8 matrix peak, and the measured GEMM's fraction of that floor; the
    same at the FMA rate measured at the GEMM's occupancy, and at the clock measured while
    the GEMM runs."""
    fmas = RESCALE_FMA_PER_EB * M * N * (K // 32)
    floor_us = fmas * 2 / (FP32_VECTOR_TFLOPS * 1e12) * 1e6
    occ_us = fmas * 2 / (FP32_FMA_TFLOPS_AT_GEMM_OCCUPANCY * 1e12) * 1e6
    clk_tflops = FP32_VECTOR_TFLOPS * GEMM_CLOCK_GHZ / 2.4
    clk_us = fmas * 2 / (clk_tflops * 1e12) * 1e6
    ceiling_tops = 2 * M * N * K / (floor_us * 1e-6) / 1e12
    return {"fma_per_element_block": RESCALE_FMA_PER_EB, "valu_peak_tflops": FP32_VECTOR_TFLOPS,
            "floor_us": round(floor_us, 2),
            "ceiling_frac_of_int8_peak": round(ceiling_tops / INT8_PEAK_TOPS, 4),
            "gemm_frac_of_ceiling": round(floor_us / gemm_us, 4),
            "valu_tflops_at_occupancy": FP32_FMA_TFLOPS_AT_GEMM_OCCUPANCY,
            "floor_at_occupancy_us": round(occ_us, 2),
            "gemm_frac_of_floor_at_occupancy": round(occ_us / gemm_us, 4),
            "clock_ghz_under_load": GEMM_CLOCK_GHZ,
            "valu_tflops_at_that_clock": round(clk_tflops, 1),
            "floor_at_that_clock_us": round(clk_us, 2),
            "gemm_frac_of_floor_at_that_clock": round(clk_us / gemm_us, 4)}


def quant_bytes(M: int, K: int) -> int:
    """Algorithmic HBM bytes of one quantize launch: f32 activations in, the q8 buffer out."""
    import q4_q8_int8_amd as mmq
    return 4 * M * K + mmq.mmq_q8_1_bytes(M, K)


def cpu_baseline(W: dict, window_s: float = 10.0) -> dict:
    """The CPU oracle (as it stands) on the same workload: quantize, decode, f64 product."""
    import numpy as np
    import oracle
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        pool = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        pool = affinity
    threads = min(pool, affinity)   # the BLAS pool cannot run more threads than it may use
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    M, N, K = W["M"], W["N"], W["K"]
    # The whole workload (quantize + q4_K decode + float64 product) takes well under the
    # ~10 s timing window on a many-core host, so it is repeated until the window is filled.
    reps, t0 = 0, time.perf_counter()
    while True:
        q = oracle.quantize_q8_1(W["x"])
        wf = oracle.decode_q4_K(W["w"])
        C = oracle.mmq(q, wf)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= window_s:
            break
    assert np.isfinite(C).all()
    return {"value": reps * M * N * K / dt / 1e12, "unit": "TMAC/s", "cores": int(threads),
            "kind": "oracle", "cpus_in_affinity": affinity, "blas_threads": pool,
            "cpu_model": model,
            "sample": f"the full {M}x{N}x{K} workload (quantize + q4_K decode + float64 "
                      f"product) repeated {reps} times in {dt:.1f} s"}


def copy_probe(mib: int) -> int:
    """A plain device-to-device copy of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n * 4, "launches": 5}), flush=True)
    return 0


def warm(step, warmup: int, warmup_ms: float) -> int:
    """Run step(i) at least `warmup` times and for at least `warmup_ms` of wall time, then
    synchronize. Under this load the device's clocks take tens of milliseconds to settle,
    so a step count alone (a caller may ask for a handful) would leave the timed steps
    inside the ramp. Returns the number of warmup steps run."""
    import torch
    i, t0 = 0, time.perf_counter()
    while i < warmup or (time.perf_counter() - t0) * 1e3 < warmup_ms:
        step(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()   # the wall clock must see the GPU's progress
    torch.cuda.synchronize()
    return i


def measure(W: dict, R: int, steps: int, warmup: int, tile: int = 0,
            warmup_ms: float = 0.0, workspace_bytes: int = 0) -> dict:
    """Time the whole path (quantize + GEMM) on one workload; see the module docstring.
    workspace_bytes > 0 hands the GEMM a split-K workspace of that size."""
    import torch

    import q4_q8_int8_amd as mmq

    dev = torch.device("cuda:0")
    M, N, K = W["M"], W["N"], W["K"]
    stream = torch.cuda.current_stream()

    xs = [torch.from_numpy(W["x"]).to(dev) for _ in range(R)]
    w_dev = torch.from_numpy(W["w"]).to(dev)
    reps = [torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device=dev)
            for _ in range(R)]
    q8s = [torch.empty(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device=dev) for _ in range(R)]
    Cs = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(R)]
    ws = (torch.empty(workspace_bytes, dtype=torch.uint8, device=dev) if workspace_bytes > 0
          else None)

    def events():
        return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    mmq.repack_q4_K(w_dev, N, K, reps[0])   # the library's first launch loads its code object
    torch.cuda.synchronize()
    ev_r0, ev_r1 = events()
    ev_r0.record(stream)
    for r in range(R):
        mmq.repack_q4_K(w_dev, N, K, reps[r])
    ev_r1.record(stream)
    torch.cuda.synchronize()
    repack_us = ev_r0.elapsed_time(ev_r1) * 1e3 / R

    def quant(r):
        mmq.quantize_q8_1(xs[r], M, K, q8s[r])

    def gemm(r):
        mmq.mmq_q4K_q8_1_ex(M, N, K, q8s[r], reps[r], Cs[r], force_tile=tile, workspace=ws)

    def step(i):
        quant(i % R)
        gemm(i % R)

    warmup_run = warm(step, warmup, warmup_ms)
    plan = mmq.mmq_last_kernel()

    # The timed region: exactly `steps` steps of the whole path between synchronizations,
    # with one pair of HIP events on the launch stream around it (events between the
    # kernels would add their own packets and gaps to every step).
    ev0, ev1 = events()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_gpu_ms = ev0.elapsed_time(ev1)

    # Per-kernel average launch durations: `steps` back-to-back launches of one kernel
    # between one pair of HIP events, the inputs rotating as in the steps (R copies of a
    # GEMM's inputs and output exceed the last-level cache, so no launch reuses another's
    # data).
    def kernel_avg_ms(launch):
        e0, e1 = events()
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            launch(i % R)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    q_ms, g_ms = kernel_avg_ms(quant), kernel_avg_ms(gemm)

    # The same steps replayed from a HIP graph (one captured step per rotation set): the
    # GPU time of a step without the host's per-launch cost, which dominates at small M.
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for r in range(R):
                step(r)
    stream.wait_stream(cs)
    reps_g = max(1, steps // R)
    for _ in range(2):
        g.replay()
    e0, e1 = events()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps_g):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_step_us = e0.elapsed_time(e1) * 1e3 / (reps_g * R)
    del g
    # The GEMM alone, replayed the same way: its GPU time without the host's launch cost,
    # which sets the back-to-back figure of the smallest kernels.
    g = torch.cuda.CUDAGraph()
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for r in range(R):
                gemm(r)
    stream.wait_stream(cs)
    for _ in range(2):
        g.replay()
    e0, e1 = events()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps_g):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_gemm_us = e0.elapsed_time(e1) * 1e3 / (reps_g * R)
    del g
    del xs, reps, q8s, Cs
    torch.cuda.empty_cache()
    return {"ms_per_step": wall * 1e3 / steps, "step_gpu_us": region_gpu_ms * 1e3 / steps,
            "gemm_us": g_ms * 1e3, "quant_us": q_ms * 1e3, "repack_us": repack_us, "plan": plan,
            "graph_step_us": graph_step_us,
            "graph_gemm_us": graph_gemm_us, "warmup_run": warmup_run}


def measure_fused(W: dict, R: int, steps: int, warmup: int) -> dict:
    """Time mmq_q4K_f32 (few tokens: the GEMM quantizes its own activations) as measure()
    times the two-kernel step: `steps` back-to-back launches between one pair of HIP events,
    and the same launches replayed from a HIP graph."""
    import torch

    import q4_q8_int8_amd as mmq

    dev = torch.device("cuda:0")
    M, N, K = W["M"], W["N"], W["K"]
    stream = torch.cuda.current_stream()
    xs = [torch.from_numpy(W["x"]).to(dev) for _ in range(R)]
    w_dev = torch.from_numpy(W["w"]).to(dev)
    reps = [torch.empty(mmq.mmq_q4K_repacked_bytes(N, K), dtype=torch.uint8, device=dev)
            for _ in range(R)]
    for r in range(R):
        mmq.repack_q4_K(w_dev, N, K, reps[r])
    Cs = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(R)]

    def call(r):
        mmq.mmq_q4K_f32(M, N, K, xs[r], reps[r], Cs[r])

    for i in range(warmup):
        call(i % R)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        call(i % R)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for r in range(R):
                call(r)
    stream.wait_stream(cs)
    reps_g = max(1, steps // R)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps_g):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / (reps_g * R)
    del g, xs, reps, Cs
    torch.cuda.empty_cache()
    return {"us": us, "graph_us": graph_us}


def measure_f16(W: dict, R: int, steps: int, warmup: int) -> dict:
    """Time the f16 comparator path on one workload: f32 -> f16 conversion of the activations,
    q4_K -> f16 dequantization of the weights, and the f16 GEMM, each as `steps`
    back-to-back launches between one pair of HIP events (inputs rotating over R copies as in
    measure()), and the two whole paths: per call (convert + dequantize + GEMM, the weights
    kept in q4_K) and with the weights resident in f16 (convert + GEMM)."""
    import torch

    import q4_q8_int8_amd as mmq

    dev = torch.device("cuda:0")
    M, N, K = W["M"], W["N"], W["K"]
    stream = torch.cuda.current_stream()
    xs = [torch.from_numpy(W["x"]).to(dev) for _ in range(R)]
    ws = [torch.from_numpy(W["w"]).to(dev) for _ in range(R)]
    x16 = [torch.empty(M * K, dtype=torch.float16, device=dev) for _ in range(R)]
    w16 = [torch.empty(N * K, dtype=torch.float16, device=dev) for _ in range(R)]
    Cs = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(R)]

    def conv(r):
        mmq.convert_f32_f16(xs[r], M, K, x16[r])

    def deq(r):
        mmq.dequantize_q4_K_f16(ws[r], N, K, w16[r])

    def gemm(r):
        mmq.gemm_f16(M, N, K, x16[r], w16[r], Cs[r])

    def per_call(r):
        conv(r)
        deq(r)
        gemm(r)

    def resident(r):
        conv(r)
        gemm(r)

    def avg_us(launch):
        for i in range(warmup):
            launch(i % R)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            launch(i % R)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    out = {"convert_us": avg_us(conv), "dequant_us": avg_us(deq), "gemm_us": avg_us(gemm),
           "per_call_us": avg_us(per_call), "resident_us": avg_us(resident)}
    del xs, ws, x16, w16, Cs
    torch.cuda.empty_cache()
    return out


def f16_summary(M: int, N: int, K: int, f: dict) -> dict:
    """The comparator's times, throughput and HBM fractions of its two own kernels."""
    macs = M * N * K
    conv_bytes = 6 * M * K                       # f32 in, f16 out
    deq_bytes = N * (K // 256) * 144 + 2 * N * K  # q4_K in, f16 out
    return {"path": "f32->f16 convert + q4_K->f16 dequantize + f16 MFMA GEMM (f32 out)",
            "dtype": "f16",
            "convert_us": round(f["convert_us"], 2),
            "convert_hbm_frac": round(conv_bytes / (f["convert_us"] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "dequant_us": round(f["dequant_us"], 2),
            "dequant_hbm_frac": round(deq_bytes / (f["dequant_us"] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "gemm_us": round(f["gemm_us"], 2),
            "gemm_tmacs": round(macs / (f["gemm_us"] * 1e-6) / 1e12, 2),
            "gemm_f16_peak_frac": round(2 * macs / (f["gemm_us"] * 1e-6) / 1e12 / F16_PEAK_TFLOPS, 4),
            "per_call_us": round(f["per_call_us"], 2),
            "per_call_tmacs": round(macs / (f["per_call_us"] * 1e-6) / 1e12, 2),
            "weights_resident_us": round(f["resident_us"], 2),
            "weights_resident_tmacs": round(macs / (f["resident_us"] * 1e-6) / 1e12, 2)}


def gemm_bytes(M: int, N: int, K: int) -> int:
    """Algorithmic HBM bytes of one GEMM launch: the q8 buffer and the repacked weights in,
    C out."""
    import q4_q8_int8_amd as mmq
    return mmq.mmq_q8_1_bytes(M, K) + mmq.mmq_q4K_repacked_bytes(N, K) + 4 * M * N


def rotation(M: int, N: int, K: int, r_min: int) -> int:
    """Input/output sets to rotate over so that one pass over them (at least 512 MiB, at most
    64 sets) exceeds the 256 MB last-level cache: with few tokens a set is little more than
    the weights, and 8 of them would stay cache-resident."""
    per_set = 5.6 * M * K + (N + 31) // 32 * (K // 256) * 4608 + 4 * M * N
    return int(min(64, max(r_min, -(-(512 << 20) // per_set))))


DECODE_SHAPES = [(1, 4096, 4096), (2, 4096, 4096), (4, 4096, 4096), (5, 4096, 4096),
                 (8, 4096, 4096), (12, 4096, 4096), (16, 4096, 4096), (8, 8192, 4096),
                 (16, 8192, 4096), (1, 11008, 4096), (4, 11008, 4096), (8, 11008, 4096),
                 (16, 11008, 4096), (1, 4096, 11008), (16, 4096, 11008)]


def decode_m1(args) -> dict:
    """One token against the q-proj weights (1 x 4096 x 4096), as --decode times it: not the
    benchmark's workload, a second line of sight on the few-token kernels."""
    import synth
    import q4_q8_int8_amd as mmq
    M, N, K = 1, 4096, 4096
    W = {"M": M, "N": N, "K": K, "x": synth.activations("normal_outliers", M, K, 1500 + M),
         "w": synth.q4k_weights("fit", N, K, 2004)[0]}
    R = rotation(M, N, K, args.rotate)
    t = measure(W, R, args.steps, args.warmup, mmq.MMQ_TILE_GEMV)
    fu = measure_fused(W, R, args.steps, args.warmup)
    wbytes = mmq.mmq_q4K_repacked_bytes(N, K)
    return {"shape": "1 x 4096 x 4096", "rotate": R,
            "fused_call_graph_us": round(fu["graph_us"], 2),
            "gemv_graph_us": round(t["graph_gemm_us"], 2),
            "gemv_weights_tbps": round(wbytes / (t["graph_gemm_us"] * 1e-6) / 1e12, 2),
            "quantize_then_gemv_graph_us": round(t["graph_step_us"], 2)}


def decode(args) -> int:
    """Few-token products (decode shapes of a 7B layer): each shape under the decode tile
    and the skinny tile, and through the fused call, with inputs rotated beyond the
    last-level cache. One JSON line per shape; --shape M,N,K runs one shape only."""
    import synth
    import q4_q8_int8_amd as mmq
    shapes = DECODE_SHAPES
    if args.shape:
        shapes = [tuple(int(v) for v in args.shape.split(","))]
    for M, N, K in shapes:
        x = synth.activations("normal_outliers", M, K, 1500 + M)
        w, _ = synth.q4k_weights("fit", N, K, 2004)
        W = {"M": M, "N": N, "K": K, "x": x, "w": w}
        R = rotation(M, N, K, args.rotate)
        wbytes = mmq.mmq_q4K_repacked_bytes(N, K)
        line = {"config": "decode", "M": M, "N": N, "K": K, "rotate": R}
        for tile, name in ((mmq.MMQ_TILE_GEMV, "gemv"), (mmq.MMQ_TILE_SKINNY, "skinny")):
            t = measure(W, R, args.steps, args.warmup, tile)
            line[name] = {"gemm_graph_us": round(t["graph_gemm_us"], 2),
                          "gemm_us": round(t["gemm_us"], 2),
                          "weights_tbps": round(wbytes / (t["graph_gemm_us"] * 1e-6) / 1e12, 2),
                          "step_graph_us": round(t["graph_step_us"], 2),
                          "step_us": round(t["step_gpu_us"], 2)}
        fu = measure_fused(W, R, args.steps, args.warmup)
        line["fused"] = {"graph_us": round(fu["graph_us"], 2), "us": round(fu["us"], 2)}
        print(json.dumps(line), flush=True)
    return 0


def config_line(name: str, W: dict, t: dict) -> dict:
    """One JSON line of the per-config table: throughput, peak and HBM fractions."""
    M, N, K = W["M"], W["N"], W["K"]
    macs = M * N * K
    g = t["gemm_us"] * 1e-6
    return {"config": name, "M": M, "N": N, "K": K, "tile": t["plan"]["tile"],
            "grid": t["plan"]["grid"],
            "gemm_us": round(t["gemm_us"], 2), "gemm_tmacs": round(macs / g / 1e12, 2),
            "gemm_us_per_gmac": round(t["gemm_us"] / (macs / 1e9), 4),
            "int8_peak_frac": round(2 * macs / g / 1e12 / INT8_PEAK_TOPS, 4),
            "gemm_hbm_frac": round(gemm_bytes(M, N, K) / g / (HBM_PEAK_GBS * 1e9), 4),
            "quant_us": round(t["quant_us"], 2),
            "quant_hbm_frac": round(quant_bytes(M, K) / (t["quant_us"] * 1e-6)
                                    / (HBM_PEAK_GBS * 1e9), 4),
            "step_us": round(t["step_gpu_us"], 2),
            "path_tmacs": round(macs / (t["step_gpu_us"] * 1e-6) / 1e12, 2),
            "graph_step_us": round(t["graph_step_us"], 2),
            "graph_path_tmacs": round(macs / (t["graph_step_us"] * 1e-6) / 1e12, 2),
            "graph_gemm_us": round(t["graph_gemm_us"], 2),
            "rotate": t["rotate"]}


def q6k_line(name: str, W: dict, R: int, steps: int, warmup: int) -> dict:
    """The q6_K x q8_1 product on a workload's shape (q6_K weights fitted to the same kind
    of synthetic matrix): `steps` back-to-back launches of its GEMM (the guard's tile) between
    one pair of HIP events, the inputs rotating over R sets."""
    import torch

    import synth
    import q4_q8_int8_amd as mmq

    dev = torch.device("cuda:0")
    M, N, K = W["M"], W["N"], W["K"]
    stream = torch.cuda.current_stream()
    w6, _ = synth.q6k_weights("fit", N, K, 2006)
    w_dev = torch.from_numpy(w6).to(dev)
    x = torch.from_numpy(W["x"]).to(dev)
    reps = [torch.empty(mmq.mmq_q6K_repacked_bytes(N, K), dtype=torch.uint8, device=dev)
            for _ in range(R)]
    q8s = [torch.empty(mmq.mmq_q8_1_bytes(M, K), dtype=torch.uint8, device=dev) for _ in range(R)]
    Cs = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(R)]
    for r in range(R):
        mmq.repack_q6_K(w_dev, N, K, reps[r])
        mmq.quantize_q8_1(x, M, K, q8s[r])

    def gemm(i):
        mmq.mmq_q6K_q8_1(M, N, K, q8s[i % R], reps[i % R], Cs[i % R])

    warm(gemm, warmup, 100.0)
    plan = mmq.mmq_last_kernel()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        gemm(i)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    macs = M * N * K
    return {"config": name, "M": M, "N": N, "K": K,
            "q6_K": {"tile": plan["tile"], "grid": plan["grid"], "gemm_us": round(us, 2),
                     "gemm_tmacs": round(macs / (us * 1e-6) / 1e12, 2),
                     "int8_peak_frac": round(2 * macs / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4),
                     "repacked_bytes": mmq.mmq_q6K_repacked_bytes(N, K)}}


def sweep(args) -> int:
    """Every configuration (and each tile the guard allows), then the 7-projection prefill:
    one JSON line each. Not the headline benchmark line; see the profiles."""
    import synth
    import q4_q8_int8_amd as mmq
    names = ["tiny", "qproj", "gateup", "down"] + [f"sweep_m{m}" for m in synth.SWEEP_M] \
        + list(synth.SHARE8)
    if args.config:
        names = [n for n in args.config.split(",") if n]
    times = {}
    for name in names:
        W = synth.workload(name)
        R = rotation(W["M"], W["N"], W["K"], args.rotate)
        tiles = [mmq.MMQ_TILE_LARGE, mmq.MMQ_TILE_SMALL]
        if W["M"] <= 2048:
            tiles[1:1] = [mmq.MMQ_TILE_HALF, mmq.MMQ_TILE_MEDIUM]
        if W["M"] <= 512:
            tiles.append(mmq.MMQ_TILE_SKINNY)
        if W["M"] <= mmq.GEMV_MAX_M:
            tiles.append(mmq.MMQ_TILE_GEMV)
        for tile in tiles:
            t = measure(W, R, args.steps, args.warmup, tile)
            t["rotate"] = R
            times[(name, tile)] = t
            print(json.dumps(config_line(name, W, t)), flush=True)
        # the guard's choice when it may split K over workgroups (a caller's workspace)
        wsb = mmq.mmq_workspace_bytes(W["M"], W["N"], W["K"])
        if wsb > 0:
            t = measure(W, R, args.steps, args.warmup, mmq.MMQ_TILE_AUTO, workspace_bytes=wsb)
            t["rotate"] = R
            times[(name, "split")] = t
            line = config_line(name, W, t)
            line.update({"workspace_bytes": wsb, "splits": t["plan"].get("splits")})
            print(json.dumps(line), flush=True)
        if name in ("tiny", "qproj"):
            print(json.dumps(q6k_line(name, W, R, args.steps, args.warmup)), flush=True)
        if W["M"] <= 128:
            fu = measure_fused(W, R, args.steps, args.warmup)
            macs = W["M"] * W["N"] * W["K"]
            print(json.dumps({"config": name, "M": W["M"], "N": W["N"], "K": W["K"],
                              "fused": {"us": round(fu["us"], 2),
                                        "graph_us": round(fu["graph_us"], 2),
                                        "tmacs": round(macs / (fu["us"] * 1e-6) / 1e12, 2)}}),
                  flush=True)
        if not args.no_f16:
            f = measure_f16(W, R, args.steps, args.warmup)
            times[(name, "f16")] = f
            print(json.dumps({"config": name, "M": W["M"], "N": W["N"], "K": W["K"],
                              "comparator_f16": f16_summary(W["M"], W["N"], W["K"], f)}),
                  flush=True)
        del W
    if args.config:
        return 0
    # 7-projection prefill of a 32-layer 7B at 2048 tokens, GEMM-only: per layer q, k, v, o
    # are q-proj shaped, gate and up gate/up shaped, down down shaped; three K=4096
    # activations (attention input, attention output, FFN input) and one K=11008 one are
    # quantized. Each product takes its faster tile.
    best = {n: min((t for (c, k), t in times.items() if c == n and k not in ("f16", "split")),
                   key=lambda t: t["gemm_us"])
            for n in ("qproj", "gateup", "down")}
    layer_gemm = 4 * best["qproj"]["gemm_us"] + 2 * best["gateup"]["gemm_us"] \
        + best["down"]["gemm_us"]
    layer_quant = 3 * best["qproj"]["quant_us"] + best["down"]["quant_us"]
    macs = 32 * (4 * 2048 * 4096 * 4096 + 2 * 2048 * 4096 * 11008 + 2048 * 11008 * 4096)
    total_us = 32 * (layer_gemm + layer_quant)
    print(json.dumps({"config": "prefill_7shape_32layer", "tokens": 2048,
                      "tok_per_s": round(2048 / (total_us * 1e-6), 1),
                      "ms": round(total_us * 1e-3, 3), "gemm_ms": round(32 * layer_gemm * 1e-3, 3),
                      "quant_ms": round(32 * layer_quant * 1e-3, 3),
                      "tmacs": round(macs / (total_us * 1e-6) / 1e12, 2),
                      "note": "sum of per-kernel averages of the 3 distinct shapes, x32 layers; "
                              "GEMM-only prefill, not whole-model"}), flush=True)
    if not args.no_f16:
        # the same prefill on the f16 comparator: per call (weights dequantized each product)
        # and with the weights resident in f16
        f16 = {n: times[(n, "f16")] for n in ("qproj", "gateup", "down")}
        layer_gemm = 4 * f16["qproj"]["gemm_us"] + 2 * f16["gateup"]["gemm_us"] \
            + f16["down"]["gemm_us"]
        layer_deq = 4 * f16["qproj"]["dequant_us"] + 2 * f16["gateup"]["dequant_us"] \
            + f16["down"]["dequant_us"]
        layer_conv = 3 * f16["qproj"]["convert_us"] + f16["down"]["convert_us"]
        for mode, layer in (("per_call", layer_gemm + layer_deq + layer_conv),
                            ("weights_resident", layer_gemm + layer_conv)):
            total = 32 * layer
            print(json.dumps({"config": "prefill_7shape_32layer_f16", "mode": mode,
                              "tokens": 2048, "tok_per_s": round(2048 / (total * 1e-6), 1),
                              "ms": round(total * 1e-3, 3),
                              "tmacs": round(macs / (total * 1e-6) / 1e12, 2),
                              "note": "f16 comparator, sum of per-kernel averages x32 layers; "
                                      "per_call dequantizes every weight matrix"}),
                  flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Under sustained quantize+GEMM steps the device needs ~50 ms (~400 q-proj steps) to
    # settle: the first steps take up to 1.5x the steady-state time. The default warmup
    # covers that; the timed steps then measure the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--warmup-ms", type=float, default=300.0,
                    help="also warm up for at least this much wall time (the clocks' ramp)")
    ap.add_argument("--rotate", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    ap.add_argument("--no-f16", action="store_true",
                    help="skip the f16 comparator path's timing")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the one-token (decode) entry of the benchmark line")
    ap.add_argument("--decode", action="store_true",
                    help="few-token shapes: vector-ALU vs skinny tile vs fused call, one JSON "
                         "line per shape")
    ap.add_argument("--shape", default="", metavar="M,N,K",
                    help="with --decode: one shape only")
    ap.add_argument("--sweep", action="store_true",
                    help="per-config table (one JSON line per config and tile) instead of the "
                         "benchmark line")
    ap.add_argument("--config", default="", metavar="NAMES",
                    help="with --sweep: only these configurations (comma-separated names)")
    args = ap.parse_args()
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode. It would "
              "shard by splitting the output features or the tokens over the GPUs, each "
              "running the same kernels on its share (--sweep measures the 8-way shares)",
              file=sys.stderr)
        return 2

    import torch

    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.sweep:
        return sweep(args)
    if args.decode:
        return decode(args)

    W = synth.workload("qproj")
    M, N, K = W["M"], W["N"], W["K"]
    R = max(1, args.rotate)
    t = measure(W, R, args.steps, args.warmup, warmup_ms=args.warmup_ms)
    plan = t["plan"]
    macs = M * N * K
    ms_per_step = t["ms_per_step"]
    gemm_s = t["gemm_us"] * 1e-6
    q_us = t["quant_us"]
    achieved_tops = 2.0 * macs / gemm_s / 1e12
    value = macs / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "q4_K x q8_1 MMQ TMAC/s (and us/GMAC) at M=2048,K=4096,N=4096",
        "value": round(value, 2),
        "unit": "TMAC/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / PAGES_QPROJ_TMACS, 2),
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "q4_K x q8_1 q-proj prefill GEMM, quantize + GEMM per step",
                   "M": M, "N": N, "K": K, "rotate": R,
                   "tile": plan["tile"], "block_m": plan["block_m"], "block_n": plan["block_n"],
                   "grid": plan["grid"], "lds_bytes": plan["lds_bytes"]},
        "roofline": {"bound": "mfma", "achieved": round(achieved_tops, 1),
                     "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                     "frac": round(achieved_tops / INT8_PEAK_TOPS, 4),
                     "traffic": measured_traffic()},
        # The GEMM's vector-ALU rescale alone, at the non-packed FP32 vector rate, bounds the
        # GEMM below the int8 matrix peak: the ceiling it implies and how close the GEMM gets.
        "epilogue_ceiling": epilogue_ceiling(M, N, K, gemm_s * 1e6),
        "us_per_gmac": round(ms_per_step * 1e3 / (macs / 1e9), 4),
        "step_gpu_us": round(t["step_gpu_us"], 2),
        "graph_step_us": round(t["graph_step_us"], 2),
        # the timed step against its two kernels' own averages, measured right after it: a
        # ratio well below 1 would mean the timed steps ran at another clock than the
        # kernels (e.g. still inside the warmup ramp)
        "step_over_kernel_sum": round(t["step_gpu_us"] / (t["quant_us"] + t["gemm_us"]), 4),
        "warmup_steps_run": t["warmup_run"],
        "gemm": {"us": round(gemm_s * 1e6, 2),
                 "tmacs": round(macs / gemm_s / 1e12, 2),
                 "us_per_gmac": round(gemm_s * 1e6 / (macs / 1e9), 4)},
        "quantize": {"us": round(q_us, 2),
                     "hbm_frac": round(quant_bytes(M, K) / (q_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
                                       4)},
        "repack_us_once": round(t["repack_us"], 2),
    }
    if not args.no_f16:
        out["comparator_f16"] = f16_summary(M, N, K, measure_f16(W, R, args.steps, args.warmup))
    if not args.no_decode:
        out["decode_m1"] = decode_m1(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
