#!/usr/bin/env python3
"""Benchmark of the forward pass of one DeepSeek-V3 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload uniform_16k]

One step is the whole hot path on one batch of seeded synthetic tokens already
resident in HBM: moe_route -> fp8_quant_1x128 -> moe_permute ->
grouped_gemm_fp8_up -> grouped_gemm_fp8_down -> moe_combine.  The expert
weights are quantised once beforehand (the offline 128x128 step), as for a
deployed layer.  Prints one JSON line (rank 0).

The default workload is the V3 layer at 16384 tokens with near-uniform expert
load, the headline case for the grouped FP8 GEMM.  ``roofline`` reports the
dominant kernel (the first expert GEMM, 2/3 of the FLOPs) against the MI355X
dense FP8 MFMA peak, timed with HIP events on the stream it runs on;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload,
and (``tiny_one_core``) on the whole tiny workload with one BLAS thread.
``measured_roofs`` measures the FP8 MFMA rate, the HBM read rate, the
direct-load stream rate and the unloaded miss latency on this GPU; ``decode``
times the 64-token workload on the same resident weights (HBM-bound); with
``--tiny``, ``tiny`` times the 256-token tiny workload (launch-bound).
``e8m0_variant`` times the same workload once more with power-of-two scales on
the hardware block-scaled MFMA (weights requantised with that rule, outside
the timed region); the headline ``value`` is the FP32-scale method.
``backward`` times the layer's backward (FP8 Dgrad and Wgrad, SwiGLU
recomputed from the forward's FP8 cache) for one output gradient of the same
batch, after a training forward outside the timed region.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import routing_fp8_grouped_amd as moe  # noqa: E402
from routing_fp8_grouped_amd import configs, inputs, profiling  # noqa: E402

METRIC = "MoE-layer tokens/s at d=7168,E=256,k=8; FP8 grouped-GEMM % of MFMA peak"
FP8_PEAK_TFLOPS = 5000.0      # MI355X dense E4M3 MFMA
HBM_PEAK_GBS = 8000.0
STAGES = ["route", "quant", "permute", "gemm_up", "gemm_down", "combine"]
BWD_STAGES = ["combine_bwd", "dgrad_w2", "swiglu_bwd", "dgrad_w13", "regroup", "wgrad_w2", "wgrad_w13"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def read_traffic(workload, kernel):
    """HBM bytes per launch of the first expert GEMM from the committed PMC
    summary, if it was taken on this kernel and its current source (else
    None)."""
    path = os.path.join(ROOT, "profiles", f"grouped_gemm_up_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel", profiling.TILED) != kernel:
        return None
    if vals.get("kernel_source_sha256_16") != profiling.gemm_source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_weights(cfg, pow2=False):
    W = moe.MoEWeights.empty(cfg.E + 1, cfg.d, cfg.f)
    for e in range(cfg.E + 1):
        w13, w2 = inputs.expert_weights(cfg, e, "cuda")
        W.quantize_expert(e, w13, w2, pow2=pow2)
        del w13, w2
    torch.cuda.synchronize()
    return W


def cpu_baseline(cfg, n_tokens):
    """Time the oracle (as it stands) on the first n_tokens tokens of the
    workload.  The experts those tokens need are quantised by the oracle first
    (the offline step, untimed); the timed part is routing, activation
    quantisation, the experts' blocked GEMMs with SwiGLU and requantisation,
    and the combine."""
    import concurrent.futures as cf
    from oracle import layer as olayer, route as oroute
    # host cores this process may run on, and the threads numpy's BLAS uses
    # for the oracle's products (the rest of the oracle is one Python thread)
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = affinity
    cores = min(affinity, blas)
    x = inputs.activations(cfg, T=n_tokens).float().numpy()
    wg = inputs.router_weights(cfg).float().numpy()
    b = inputs.selection_bias(cfg).numpy()
    r = oroute.route(x, wg, b, cfg.G, cfg.M, cfg.k, cfg.route_scale)
    need = sorted(set(r["idx"].reshape(-1).tolist()) | {cfg.E})

    def quantize(e):
        w13, w2 = inputs.expert_weights(cfg, e, "cuda")     # the GPU run's values
        return olayer.quantize_expert(w13.float().cpu().numpy(), w2.float().cpu().numpy())

    # at most `workers` experts in flight: ~1 GB of host memory each
    workers = min(8, os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(workers) as ex:
        q = dict(zip(need, ex.map(quantize, need)))
    t0 = time.perf_counter()
    olayer.moe_layer_tokens(x, wg, b, lambda e: q[e], cfg.G, cfg.M, cfg.k, cfg.route_scale)
    dt = time.perf_counter() - t0
    out = {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
           "affinity_cores": affinity, "blas_threads": int(blas),
            "sample": f"first {n_tokens} token(s) of the {cfg.name} workload, whole layer "
                      f"({len(need)} experts incl. shared), {dt:.1f} s; expert weights "
                      "quantised by the oracle beforehand (untimed, as on the GPU); cores = "
                      "min(sched_getaffinity cores, BLAS threads): the oracle's products run "
                      "on the BLAS threads, its loops on one Python thread"}
    out["tiny_one_core"] = oracle_tiny_one_core()
    return out


def oracle_tiny_one_core(min_seconds=2.0):
    """The oracle on all 256 tokens of the tiny configuration with its BLAS
    limited to one thread: the median of repeated passes (about two seconds of
    work), expert weights quantised beforehand (untimed)."""
    from threadpoolctl import threadpool_limits
    from oracle import layer as olayer
    cfg = configs.get("tiny")
    x = inputs.activations(cfg).float().numpy()
    wg = inputs.router_weights(cfg).float().numpy()
    b = inputs.selection_bias(cfg).numpy()
    q = {}
    for e in range(cfg.E + 1):
        w13, w2 = inputs.expert_weights(cfg, e, "cuda")     # the GPU leg's values
        q[e] = olayer.quantize_expert(w13.float().cpu().numpy(), w2.float().cpu().numpy())
    times = []
    with threadpool_limits(1):
        while sum(times) < min_seconds or len(times) < 3:
            t0 = time.perf_counter()
            olayer.moe_layer_tokens(x, wg, b, lambda e: q[e], cfg.G, cfg.M, cfg.k, cfg.route_scale)
            times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": cfg.T / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"all {cfg.T} tokens of the tiny workload (d {cfg.d}, {cfg.E}+1 experts, k {cfg.k}), "
                      f"BLAS limited to one thread; median of {len(times)} passes, {dt * 1e3:.1f} ms each"}


def tiny_leg(steps, warmup):
    """The tiny configuration (256 tokens, d 256, 16 routed experts): a layer
    whose kernels are each far below a microsecond of work, so its time is the
    launches' (eager, and replayed from a HIP graph)."""
    cfg = configs.get("tiny")
    x, wg, b = (t.cuda() for t in inputs.host_inputs(cfg))
    W = build_weights(cfg)
    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.f, cfg.route_scale)
    for _ in range(warmup):
        layer.forward(x, wg, b, W)
    torch.cuda.synchronize()
    ms, st = timed_steps(layer, x, wg, b, W, steps)
    graph_ms = timed_graph(layer, x, wg, b, W, steps)
    log(f"tiny: {ms:.3f} ms/step eager, {graph_ms:.3f} ms/step from a graph; stages "
        + ", ".join(f"{k} {v:.3f}" for k, v in st.items()))
    return {"workload": cfg.name, "tokens": cfg.T, "ms_per_step": ms, "tokens_per_s": cfg.T / (ms * 1e-3),
            "graph_ms_per_step": graph_ms, "graph_tokens_per_s": cfg.T / (graph_ms * 1e-3),
            "stages_ms": st,
            "note": "launch-bound: each of the six stages is one to a few small kernels; the graph "
                    "replay removes the host's launch gaps"}


def timed_steps(layer, x, wg, b, W, steps):
    """Wall time per step over ``steps`` layer steps (bracketed by device
    synchronisations) and per-stage times from HIP events recorded on the
    stream the kernels run on."""
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(STAGES) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        marks = ev[s]
        marks[0].record(stream)
        it = iter(marks[1:])
        layer.forward(x, wg, b, W, mark=lambda name: next(it).record(stream))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage_ms = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
                for i, name in enumerate(STAGES)}
    return (t1 - t0) * 1e3 / steps, stage_ms


def gini(counts):
    """Gini coefficient of the routed experts' row counts (0: equal loads)."""
    c = np.sort(np.asarray(counts, np.float64))
    n = len(c)
    return float(2.0 * np.sum(np.arange(1, n + 1) * c) / (n * c.sum()) - (n + 1.0) / n) if c.sum() > 0 else 0.0


def timed_graph(layer, x, wg, b, W, steps):
    """Milliseconds per forward replayed from a HIP graph (the same launches
    captured once; no launch gaps), bracketed by device synchronisations."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, wg, b, W)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, wg, b, W)
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    del g
    return ms


def timed_backward(layer, dout, Wt, steps):
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(BWD_STAGES) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record(stream)
        it = iter(ev[s][1:])
        layer.backward(dout, Wt, mark=lambda name: next(it).record(stream))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage_ms = {name: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)]))
                for i, name in enumerate(BWD_STAGES)}
    return (t1 - t0) * 1e3 / steps, stage_ms


def measured_roofs(reps=5):
    """The FP8 MFMA issue rate and the HBM read rate this GPU sustains, from
    the library's two measurement kernels (moe_roof_fp8_mfma,
    moe_roof_hbm_read), timed with HIP events on the launch stream; the median
    of ``reps`` runs."""
    import ctypes
    lib = moe._lib.load()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg_mfma, iters = 2 * cus, 20000
    sink = torch.empty(max(wg_mfma, 8 * cus) * 256, dtype=torch.float32, device="cuda")
    buf = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")     # 16x the last-level cache
    buf.fill_(1)

    def timed(call, reps=reps):
        ms = []
        for _ in range(reps + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            moe._lib.check("roof", call())
            b.record(stream)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms[1:]))     # the first run warms up

    ms_mfma = timed(lambda: lib.moe_roof_fp8_mfma(wg_mfma, iters, ctypes.c_void_p(sink.data_ptr()), sp))
    flop = wg_mfma * 4 * iters * 8 * 65536
    ms_read = timed(lambda: lib.moe_roof_hbm_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), 2 * cus,
                                                  ctypes.c_void_p(sink.data_ptr()), sp))
    # the expert GEMMs' weight-load pattern (rows of 7168 bytes, direct loads
    # into per-wave LDS rings, one workgroup of 8 waves per CU) with 1, 2 and
    # 4 blocks of 4 KB in flight per wave
    K = 7168
    dma_bytes = (buf.numel() // (32 * K)) * 32 * K
    dma = {}
    for ahead in (1, 2, 4):
        ms = timed(lambda: lib.moe_roof_dma_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(), K, ahead, cus,
                                                 ctypes.c_void_p(sink.data_ptr()), sp))
        dma[ahead] = dma_bytes / (ms * 1e-3) / 1e9
    # latency of a load that misses every cache: a chain of dependent loads in
    # random order over the buffer's first 2 GiB, one entry per 128-byte line;
    # streaming the other half afterwards evicts the chain from the caches
    lines = 1 << 24
    nxt = buf.view(torch.int32)[: lines * 32]
    perm = torch.randperm(lines, device="cuda", generator=torch.Generator(device="cuda").manual_seed(7))
    nxt[perm * 32] = (torch.roll(perm, -1) * 32).to(torch.int32)
    del perm
    half = buf[(lines * 128):]
    lib.moe_roof_hbm_read(ctypes.c_void_p(half.data_ptr()), half.numel(), 2 * cus,
                          ctypes.c_void_p(sink.data_ptr()), sp)
    # each run continues the chain where the previous one stopped, so every
    # run reads lines no run has touched since the eviction
    steps, pos, ms = 20000, 0, []
    for _ in range(4):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        moe._lib.check("roof", lib.moe_roof_hbm_latency(ctypes.c_void_p(nxt.data_ptr()), nxt.numel(), pos, steps,
                                                        ctypes.c_void_p(sink.data_ptr()), sp))
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
        pos = int(sink[:1].view(torch.int32).item())
    latency_ns = float(np.median(ms[1:])) * 1e6 / steps
    del buf, sink, nxt, half
    torch.cuda.empty_cache()
    per_cu = dma[1] * 1e9 / cus                     # bytes per second per CU, one block per wave in flight
    return {"fp8_mfma_tflops": flop / (ms_mfma * 1e-3) / 1e12,
            "hbm_read_gbs": (4 << 30) / (ms_read * 1e-3) / 1e9,
            "hbm_dma_gbs": {str(a): v for a, v in dma.items()},
            "hbm_latency_ns": latency_ns,
            "lines_in_flight_per_cu": per_cu * latency_ns * 1e-9 / 128,
            "note": "moe_roof_fp8_mfma: 8 independent FP8 MFMA chains per wave, no memory traffic, "
                    f"{wg_mfma} workgroups x 4 waves; moe_roof_hbm_read: non-temporal 16-byte loads over "
                    f"a 4 GiB buffer, a contiguous share per workgroup, {2 * cus} workgroups; "
                    f"moe_roof_dma_read: rows of {K} bytes, 8 waves per CU, each streaming 32 rows into its "
                    "LDS ring with 1, 2 or 4 K blocks of 4 KB in flight; moe_roof_hbm_latency: "
                    f"{steps} dependent loads in random order over 2 GiB (unloaded latency); "
                    "lines_in_flight_per_cu: the DMA rate with one block in flight per wave, per CU, "
                    "times that latency over 128 bytes (Little's law; a lower bound, since the latency "
                    f"under load is higher); median of {reps} runs each"}


def decode_leg(W, roofs, steps, warmup):
    """The decode workload (64 tokens at the V3 shape) on the same resident FP8
    weights: layer time, the HBM rate of the bytes the method must move, and
    the roofline of its dominant kernel (the first expert GEMM, HBM-bound)."""
    cfg = configs.get("decode_64")
    x, wg, b = (t.cuda() for t in inputs.host_inputs(cfg))
    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.f, cfg.route_scale)
    for _ in range(warmup):
        layer.forward(x, wg, b, W)
    torch.cuda.synchronize()
    ms, st = timed_steps(layer, x, wg, b, W, steps)
    # cold: each step after a 1 GiB write has evicted the 256 MB last-level
    # cache (the weights are 36x that, so cold and warm should agree)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    cold = []
    for i in range(max(3, steps // 2)):
        flush.fill_(i & 0xFF)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        layer.forward(x, wg, b, W)
        e.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(e))
    del flush
    cold_ms = float(np.median(cold))
    counts = np.bincount(layer.idx.cpu().numpy().reshape(-1), minlength=cfg.E)
    touched = int((counts > 0).sum()) + 1
    d, f = cfg.d, cfg.f
    w13_b = 2 * f * d + (2 * f // 128) * (d // 128) * 4
    w2_b = d * f + (d // 128) * (f // 128) * 4
    layer_bytes = touched * (w13_b + w2_b) + cfg.E * d * 2 + cfg.E * 4 + 2 * cfg.T * d * 2
    up_bytes = touched * w13_b + cfg.T * (d + d // 128 * 4) + cfg.rows * (f + f // 128 * 4)
    up_s = st["gemm_up"] * 1e-3
    layer_gbs = layer_bytes / (ms * 1e-3) / 1e9
    up_gbs = up_bytes / up_s / 1e9
    log(f"decode_64: {ms:.3f} ms/step (cold {cold_ms:.3f}), {touched} experts touched, layer "
        f"{layer_gbs:.0f} GB/s; stages " + ", ".join(f"{k} {v:.3f}" for k, v in st.items()))
    return {
        "workload": cfg.name, "tokens": cfg.T, "ms_per_step": ms, "tokens_per_s": cfg.T / (ms * 1e-3),
        "stages_ms": st, "experts_touched": touched, "algorithmic_bytes": layer_bytes,
        "hbm_gbs": layer_gbs, "hbm_frac_of_peak": layer_gbs / HBM_PEAK_GBS,
        "hbm_frac_of_measured": layer_gbs / roofs["hbm_read_gbs"],
        "cold_ms_per_step": cold_ms, "cold_hbm_gbs": layer_bytes / (cold_ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": up_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": up_gbs / HBM_PEAK_GBS, "measured_peak": roofs["hbm_read_gbs"],
                     "frac_of_measured": up_gbs / roofs["hbm_read_gbs"],
                     "kernel": "grouped_gemm_fp8_up (grouped_gemm_small_kernel<true, false>)",
                     "algorithmic_bytes_per_launch": up_bytes, "avg_launch_ms": st["gemm_up"],
                     "traffic": read_traffic(cfg.name, profiling.STREAMING)},
        "note": "algorithmic bytes: each touched expert's W1, W3, W2 codes and scales once, the "
                "router weights, the token rows in and the output out; the same resident weights "
                "as the headline workload (same shapes and distribution); cold: the median of single "
                "steps each after a 1 GiB write that evicts the last-level cache",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="uniform_16k", choices=sorted(configs.CONFIGS))
    ap.add_argument("--dispatch", action="store_true",
                    help="copy the FP8 rows into grouped order instead of gathering in the GEMM")
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-e8m0", action="store_true",
                    help="skip the timing of the power-of-two (E8M0) scale variant")
    ap.add_argument("--no-backward", action="store_true", help="skip the timing of the backward")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode_64 leg")
    ap.add_argument("--no-roofs", action="store_true", help="skip the measured roofs")
    ap.add_argument("--tiny", action="store_true",
                    help="also time the tiny workload (off by default: its expert GEMMs run the headline's "
                         "tiled kernel, whose rocprofv3 average would then mix in their launches)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MoE layer runs on a single MI355X "
              "(no sharding or collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    cfg = configs.get(args.workload)
    torch.cuda.set_device(0)
    log(f"workload {cfg.name}: T={cfg.T} d={cfg.d} E={cfg.E}+1 G={cfg.G} M={cfg.M} k={cfg.k} f={cfg.f}")
    x, wg, b = (t.cuda() for t in inputs.host_inputs(cfg))
    W = build_weights(cfg)
    layer = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.f, cfg.route_scale,
                         dispatch=args.dispatch)
    log("inputs and FP8 weights resident")

    # A plain copy of known size, outside the timed region: its FETCH_SIZE /
    # WRITE_SIZE counters calibrate the GEMM's.
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")      # 1 GiB
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)                                        # reads 1 GiB, writes 1 GiB
    torch.cuda.synchronize()
    del src, dst

    # the measured roofs and the decode leg first, on a GPU that has run nothing
    # heavy yet (the decode leg uses the same resident weights)
    roofs = None if args.no_roofs else measured_roofs()
    if roofs is not None:
        log(f"measured roofs: FP8 MFMA {roofs['fp8_mfma_tflops']:.0f} TFLOP/s, "
            f"HBM read {roofs['hbm_read_gbs']:.0f} GB/s; weight-pattern direct loads "
            + ", ".join(f"{v:.0f}" for v in roofs["hbm_dma_gbs"].values())
            + f" GB/s at 1, 2, 4 blocks in flight; load latency {roofs['hbm_latency_ns']:.0f} ns; "
            f"≥ {roofs['lines_in_flight_per_cu']:.0f} lines in flight per CU")
    decode = None
    if not args.no_decode and cfg.name != "decode_64":
        decode = decode_leg(W, roofs or {"hbm_read_gbs": float("nan")}, args.steps, args.warmup)

    for _ in range(args.warmup):
        layer.forward(x, wg, b, W)
    torch.cuda.synchronize()
    log(f"{args.warmup} warmup steps done")

    ms_per_step, stage_ms = timed_steps(layer, x, wg, b, W, args.steps)
    log(f"{args.steps} timed steps: {ms_per_step:.3f} ms/step; stages " +
        ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))
    graph_ms = timed_graph(layer, x, wg, b, W, args.steps)
    log(f"graph replay: {graph_ms:.3f} ms/step")

    counts = np.bincount(layer.idx.cpu().numpy().reshape(-1), minlength=cfg.E)
    rows = cfg.rows
    up_flop = rows * 2 * (2 * cfg.f) * cfg.d
    down_flop = rows * 2 * cfg.d * cfg.f
    up_tflops = up_flop / (stage_ms["gemm_up"] * 1e-3) / 1e12
    gemm_tflops = (up_flop + down_flop) / ((stage_ms["gemm_up"] + stage_ms["gemm_down"]) * 1e-3) / 1e12
    touched = int((counts > 0).sum()) + 1
    weight_bytes = touched * (3 * cfg.d * cfg.f + 3 * (cfg.d // 128) * (cfg.f // 128) * 4)
    # algorithmic bytes of the first expert GEMM: each touched expert's W1/W3
    # codes and scales once, the token rows once, h and its scales written once
    up_bytes = (touched * (2 * cfg.f * cfg.d + (2 * cfg.f // 128) * (cfg.d // 128) * 4)
                + cfg.T * (cfg.d + cfg.d // 128 * 4) + rows * (cfg.f + cfg.f // 128 * 4))
    up_s = stage_ms["gemm_up"] * 1e-3
    # the library streams the weights (grouped_gemm_small_kernel) when the
    # experts average at most 16 rows, and tiles otherwise
    small = rows <= 16 * (cfg.E + 1)
    up_kernel = ("grouped_gemm_fp8_up (grouped_gemm_small_kernel<true, false>)" if small
                 else "grouped_gemm_fp8_up (grouped_gemm_kernel<true, false>)")
    traffic = read_traffic(cfg.name, profiling.STREAMING if small else profiling.TILED)
    if up_flop / up_bytes >= FP8_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        roof = {"bound": "mfma", "achieved": up_flop / up_s / 1e12, "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": up_bytes / up_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roofs is not None:
        roof["measured_peak"] = roofs["fp8_mfma_tflops"] if roof["bound"] == "mfma" else roofs["hbm_read_gbs"]
        roof["frac_of_measured"] = roof["achieved"] / roof["measured_peak"]

    result = {
        "metric": METRIC,
        "value": cfg.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "d_model": cfg.d,
                   "routed_experts": cfg.E, "shared_experts": 1, "groups": cfg.G,
                   "groups_per_token": cfg.M, "topk": cfg.k, "d_ffn": cfg.f,
                   "route_scale": cfg.route_scale, "dispatch_copy": args.dispatch},
        "roofline": dict(roof, traffic=traffic,
                         kernel=up_kernel,
                         flop_per_launch=up_flop, algorithmic_bytes_per_launch=up_bytes,
                         avg_launch_ms=stage_ms["gemm_up"], tflops=up_tflops),
        "stages_ms": stage_ms,
        "grouped_gemm_tflops": gemm_tflops,
        "grouped_gemm_frac_of_fp8_peak": gemm_tflops / FP8_PEAK_TFLOPS,
        "expert_rows": {"max": int(counts.max()), "min": int(counts.min()),
                        "max_over_mean": float(counts.max() / counts.mean()), "gini": gini(counts),
                        "experts_touched": touched},
        "weights_hbm_gbs": weight_bytes / (ms_per_step * 1e-3) / 1e9,
        "graph_replay": {"ms_per_step": graph_ms, "tokens_per_s": cfg.T / (graph_ms * 1e-3),
                         "note": "the same forward captured once in a HIP graph and replayed"},
        "context": "pages: 2.788M H800 GPU-hours for the whole V3 training run; "
                   "180K H800 GPU-hours per trillion training tokens (not comparable)",
    }
    if roofs is not None:
        result["measured_roofs"] = roofs
    if decode is not None:
        result["decode"] = decode
    if args.tiny and cfg.name != "tiny":
        result["tiny"] = tiny_leg(args.steps, args.warmup)
    if not args.no_backward:
        Wt = W.transposed()
        layer.forward(x, wg, b, W, train=True)
        g = torch.Generator(device="cuda")
        g.manual_seed(cfg.seed * 7 + 3)
        dout = torch.randn(cfg.T, cfg.d, generator=g, device="cuda").to(torch.bfloat16)
        for _ in range(max(1, args.warmup // 2)):
            layer.backward(dout, Wt)
        msb, stb = timed_backward(layer, dout, Wt, args.steps)
        log(f"backward: {msb:.3f} ms/step; stages " + ", ".join(f"{k} {v:.3f}" for k, v in stb.items()))
        f_w2 = rows * 2 * cfg.d * cfg.f          # each of Dgrad W2 and Wgrad W2
        f_w13 = rows * 2 * (2 * cfg.f) * cfg.d   # each of Dgrad W13 and Wgrad W13
        dgrad_ms = stb["dgrad_w2"] + stb["dgrad_w13"]
        wgrad_ms = stb["wgrad_w2"] + stb["wgrad_w13"]
        result["backward"] = {
            "ms_per_step": msb, "stages_ms": stb, "tokens_per_s": cfg.T / (msb * 1e-3),
            "dgrad_tflops": (f_w2 + f_w13) / (dgrad_ms * 1e-3) / 1e12,
            "wgrad_tflops": (f_w2 + f_w13) / (wgrad_ms * 1e-3) / 1e12,
            "wgrad_w13_tflops": f_w13 / (stb["wgrad_w13"] * 1e-3) / 1e12,
            "weight_grad_bytes_written": 3 * (cfg.E + 1) * cfg.d * cfg.f * 4,
            "note": "dgrad_w13 includes the token-gradient gather; Wgrad writes FP32 gradients of "
                    "all experts",
        }
        del Wt, dout
        layer.__dict__.update({k: None for k in ("gu", "gus", "dy", "dyq", "dys", "dh", "dgu", "dgus",
                                                 "dgu_t", "dgu_ts", "h_t", "h_ts", "dy_t", "dy_ts", "x_t",
                                                 "x_ts", "dx_rows", "dx", "dw13", "dw2")})
        torch.cuda.empty_cache()
    if not args.no_e8m0:
        del W, layer
        torch.cuda.empty_cache()
        W8 = build_weights(cfg, pow2=True)
        layer8 = moe.MoELayer(cfg.T, cfg.d, cfg.E, cfg.G, cfg.M, cfg.k, cfg.f, cfg.route_scale,
                              dispatch=args.dispatch, scales="pow2")
        for _ in range(args.warmup):
            layer8.forward(x, wg, b, W8)
        ms8, st8 = timed_steps(layer8, x, wg, b, W8, args.steps)
        log(f"E8M0 variant: {ms8:.3f} ms/step; stages " + ", ".join(f"{k} {v:.3f}" for k, v in st8.items()))
        up8 = up_flop / (st8["gemm_up"] * 1e-3) / 1e12
        result["e8m0_variant"] = {
            "scales": "power of two, hardware block-scaled MFMA",
            "value": cfg.T / (ms8 * 1e-3), "unit": "tokens/s", "ms_per_step": ms8,
            "stages_ms": st8, "gemm_up_tflops": up8, "gemm_up_frac_of_fp8_peak": up8 / FP8_PEAK_TFLOPS,
            "grouped_gemm_tflops": (up_flop + down_flop) / ((st8["gemm_up"] + st8["gemm_down"]) * 1e-3) / 1e12,
            "kernel": ("grouped_gemm_fp8_up_e8m0 (grouped_gemm_small_kernel<true, true>)" if small
                       else "grouped_gemm_fp8_up_e8m0 (grouped_gemm_kernel<true, true>)"),
        }
        del W8, layer8
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {args.cpu_tokens} token(s)")
        result["cpu_baseline"] = cpu_baseline(cfg, args.cpu_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
