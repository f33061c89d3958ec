#!/usr/bin/env python3
"""Benchmark of the int4 MoE layer on one MI355X (gfx950).

Default workload: the 512-token prefill layer (H=2048, I=512, 256 routed
experts top-8 + 1 shared, int4 g64 weights with bf16 scale/bias), synthetic
seeded inputs already resident in HBM. One step = one call of
moe_prefill_layer: router, top-k, routing metadata, grouped gate/up + SwiGLU,
grouped down, shared expert and combine. Four copies of the packed weights
(about 1.8 GB) are used in rotation so the weights stream from HBM rather
than from the 256 MB Infinity Cache (the decode workloads rotate 32 copies,
so that even the shared expert, used every step, comes from HBM). The timed loop replays, step by step, a
HIP graph of one layer call per weight copy; an eager pass over the same
number of steps with HIP events around every launch gives the per-kernel
times.

Prints ONE JSON line on stdout (progress goes to stderr):
  value         tokens/s of the whole layer
  roofline      the dominant kernel (gate/up GEMM): algorithmic bytes or
                flops per launch / its mean duration from HIP events recorded
                on the library's stream around every launch in the timed region
                (plus that rate over the measured ceiling below)
  ceilings      measured on this device in the same run: streaming HBM read
                GB/s over a 2 GiB buffer and the bf16 MFMA loop's TFLOP/s on
                random and on nearly constant operands, each with the shader
                clock it sustained (the fractions use the random-operand rate)
  cpu_baseline  the CPU oracle timed on this host on the same workload
  roofline_mfma the matrix-core roofline (gate/up and down kernels, and the
                whole layer's expert flops) of the two long-chunk workloads
  secondary     the 2048-token Zipf-skewed prefill (bf16 MFMA fraction), the
                16384-token prompt in 4096-token chunks, and batch-1 and
                batch-4 decode (HBM GB/s of the GEMV kernels), same method

--sweep-chunks prints instead one JSON line with the 16384-token prompt
timed at chunk sizes 1024 .. 16384 (throughput against workspace size).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer prefill tokens/s at T=512/2048 + % bf16 MFMA peak; decode HBM GB/s"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6
PREFILL_KERNELS = ["router", "topk", "scan_scatter", "gemm_gateup", "gemm_down", "combine"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gateup_prefill_t512.json")
DECODE_KERNELS = ["decode_router", "decode_topk_gateup", "decode_down_combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def expert_bytes(H, I):
    """Stored bytes of one expert's gate+up and down (codes + bf16 scale + bias)."""
    mat = H * I // 2 + 2 * 2 * H * I // 64
    return 2 * mat, mat


def prefill_setup(name, copies, seed=0):
    import torch
    from int4_grouped_gemm_router_amd import binding as B
    from int4_grouped_gemm_router_amd import synth
    wl, w, x = synth.generate(name, seed=seed)
    dw = B.DeviceWeights.from_logical(w)
    dws = [dw] + [dw.clone() for _ in range(copies - 1)]
    xd = torch.from_numpy(x).cuda()
    return wl, w, x, xd, dws


def _graph_of(calls):
    """Capture `calls()` (layer launches on the current stream) into a HIP graph."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                       # warm the allocator and code objects outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    return g


def run_prefill(name, steps, warmup, copies, chunk=None, block_m=32, gemm=0):
    """Time `steps` layer calls. The step time (value) comes from replaying a
    HIP graph of `copies` consecutive layer calls (one per weight copy); the
    per-kernel durations come from HIP events recorded on the library's
    stream around every launch of an eager pass over the same steps."""
    import torch
    from int4_grouped_gemm_router_amd import binding as B
    wl, w, x, xd, dws = prefill_setup(name, copies)
    d0 = dws[0].dims
    d = B.dims(d0.H, d0.I, d0.E, d0.top_k, block_m, gemm)
    T, H, I = wl.T, wl.H, wl.I
    chunk = wl.chunk if chunk is None else chunk
    Tc = chunk if chunk else T
    chunks = -(-T // Tc)
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = B.workspace(d, Tc, B.MODE_PREFILL)
    ro = B.RouteBuffers(d, T if chunks == 1 else Tc)
    # routing of this fixed input (for the algorithmic byte count)
    B.moe_prefill_layer(d, dws[0], xd, y, T, chunk, None, ro, ws)
    torch.cuda.synchronize()
    hist = ro.hist.cpu().numpy()
    for i in range(warmup):
        B.moe_prefill_layer(d, dws[i % copies], xd, y, T, chunk, None, None, ws)
    y_eager = y.clone()

    # eager pass with events around every launch: per-kernel durations
    n_ev = 6 * chunks + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    arrays = [B._event_array(ev) for ev in events]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        B.moe_prefill_layer_profiled(d, dws[i % copies], xd, y, T, chunk, arrays[i], ws=ws)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    per = np.zeros((steps, 6 * chunks))
    for i in range(steps):
        for j in range(6 * chunks):
            per[i, j] = events[i][j].elapsed_time(events[i][j + 1])  # ms
    kern_ms = per.reshape(steps, chunks, 6).sum(axis=1).mean(axis=0) / chunks  # per launch

    # timed region: exactly `steps` graph replays, one captured layer call per
    # weight copy, replayed in rotation
    graphs = [_graph_of(lambda i=i: B.moe_prefill_layer(d, dws[i], xd, y, T, chunk, None, None, ws))
              for i in range(copies)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    graph_ok = bool(torch.equal(y, y_eager))  # every weight copy holds the same values
    if not graph_ok:
        log(f"{name}: graph replay output differs from the eager output; reporting eager timing")
        ms_step = wall_eager * 1e3 / steps

    U = int((hist > 0).sum()) if chunks == 1 else None
    gu_b, dn_b = expert_bytes(H, I)
    gate_up_flops = 2.0 * (wl.k + 1) * Tc * H * 2 * I
    expert_flops = T * (wl.k + 1) * 6.0 * H * I
    res = dict(workload=name, T=T, chunk=chunk, ms_per_step=ms_step, tokens_per_s=T / (ms_step / 1e3),
               ms_per_step_eager=wall_eager * 1e3 / steps, graph_matches_eager=graph_ok,
               kernels_us={k: float(v * 1e3) for k, v in zip(PREFILL_KERNELS, kern_ms)},
               expert_tflops=expert_flops / (ms_step / 1e3) / 1e12)
    res["mfma_frac_layer"] = res["expert_tflops"] / PEAK_BF16_TFLOPS
    gu_ms = float(kern_ms[3])
    res["gateup_tflops"] = gate_up_flops / (gu_ms / 1e3) / 1e12
    dn_ms = float(kern_ms[4])
    down_flops = 2.0 * (wl.k + 1) * Tc * H * I
    res["down_tflops"] = down_flops / (dn_ms / 1e3) / 1e12
    # matrix-core roofline of the gate/up kernel (algorithmic flops per launch
    # over its mean launch duration; HIP events on the library's stream)
    res["roofline_gateup"] = {"bound": "mfma", "achieved": res["gateup_tflops"], "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": res["gateup_tflops"] / PEAK_BF16_TFLOPS,
                              "kernel": "gemm_gateup", "per_launch_flops": gate_up_flops,
                              "mean_us": gu_ms * 1e3}
    res["roofline_down"] = {"bound": "mfma", "achieved": res["down_tflops"], "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": res["down_tflops"] / PEAK_BF16_TFLOPS,
                            "kernel": "gemm_down", "per_launch_flops": down_flops, "mean_us": dn_ms * 1e3}
    if U is not None:
        gu_bytes = (U + 1) * gu_b + T * H * 2 + (wl.k + 1) * T * I * 2
        res["touched_experts"] = U
        res["gateup_algorithmic_bytes"] = gu_bytes
        res["gateup_gbs"] = gu_bytes / (gu_ms / 1e3) / 1e9
    return res, (w, x)


def run_decode(name, steps, warmup, copies):
    """Batch-1 (or 4) decode: `steps` consecutive layer calls, each on fresh
    activations, weights rotated over `copies` copies. The timed region
    replays one HIP graph holding all `steps` calls; an eager pass with HIP
    events around every launch gives the per-kernel times."""
    import torch
    from int4_grouped_gemm_router_amd import binding as B
    from int4_grouped_gemm_router_amd import synth
    wl, w, xs = synth.generate(name, steps=steps + warmup)
    dw = B.DeviceWeights.from_logical(w)
    dws = [dw] + [dw.clone() for _ in range(copies - 1)]
    d = dw.dims
    T, H, I = wl.T, wl.H, wl.I
    xd = torch.from_numpy(xs).cuda()
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = B.workspace(d, T, B.MODE_DECODE)
    ro = B.RouteBuffers(d, T)
    for i in range(warmup):
        B.moe_decode_layer(d, dws[i % copies], xd[i], y, T, None, None, ws)
    # unique experts per step (for the byte count), from an untimed pass over the same inputs
    hists = []
    for i in range(min(steps, 64)):
        B.moe_decode_layer(d, dws[0], xd[warmup + i], y, T, None, ro, ws)
        hists.append(ro.hist.clone())
    # eager pass with events: per-kernel durations
    nk = len(DECODE_KERNELS)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
    arrays = [B._event_array(ev) for ev in events]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        B.moe_decode_layer_profiled(d, dws[i % copies], xd[warmup + i], y, T, arrays[i], ws=ws)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    y_eager = y.clone()
    per = np.array([[events[i][j].elapsed_time(events[i][j + 1]) for j in range(nk)]
                    for i in range(steps)])
    kern_ms = per.mean(axis=0)
    # timed region: one graph of all steps
    def calls():
        for i in range(steps):
            B.moe_decode_layer(d, dws[i % copies], xd[warmup + i], y, T, None, None, ws)
    g = _graph_of(calls)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    graph_ok = bool(torch.equal(y, y_eager))
    if not graph_ok:
        log(f"{name}: graph replay output differs from the eager output; reporting eager timing")
        wall = wall_eager
    U = float(np.mean([(h.cpu().numpy() > 0).sum() for h in hists]))
    gu_b, dn_b = expert_bytes(H, I)
    gemv_bytes = (U + 1) * (gu_b + dn_b)
    router_bytes = wl.E * H * 4
    # the three decode kernels move the router matrix and the selected and
    # shared experts' weights
    gemv_ms = float(kern_ms[0] + kern_ms[1] + kern_ms[2])
    ms_step = wall * 1e3 / steps
    res = dict(workload=name, T=T, steps=steps, ms_per_step=ms_step,
               ms_per_step_eager=wall_eager * 1e3 / steps, graph_matches_eager=graph_ok,
               unique_experts=U, kernels_us={k: float(v * 1e3) for k, v in zip(DECODE_KERNELS, kern_ms)},
               gemv_bytes=gemv_bytes + router_bytes,
               gemv_gbs=(gemv_bytes + router_bytes) / (gemv_ms / 1e3) / 1e9,
               step_bytes=gemv_bytes + router_bytes,
               end_to_end_gbs=(gemv_bytes + router_bytes) / (ms_step / 1e3) / 1e9)
    # HBM roofline of the step's three kernels: algorithmic bytes over their
    # summed event times; traffic = the committed FETCH_SIZE / WRITE_SIZE
    # bytes of the three launches (null if missing or stale)
    res["roofline"] = {"bound": "hbm", "achieved": res["gemv_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": res["gemv_gbs"] / PEAK_HBM_GBS, "traffic": decode_traffic(name),
                       "kernel": "+".join(DECODE_KERNELS), "per_step_bytes": res["gemv_bytes"],
                       "mean_us": gemv_ms * 1e3}
    return res


def decode_traffic(workload):
    """HBM bytes of one decode step (router, gate/up and down launches) from
    the committed traffic summaries, or None when one is missing or was taken
    from different decode sources."""
    from int4_grouped_gemm_router_amd import profiling
    total = 0.0
    for k in ("router", "gateup", "down"):
        f = os.path.join(ROOT, "profiles", f"traffic_decode_{k}_{workload}.json")
        if not os.path.exists(f):
            return None
        with open(f) as fh:
            t = json.load(fh)
        if t.get("sources_sha256") != profiling.sources_digest(profiling.DECODE_SOURCES):
            log(f"decode traffic summary {os.path.basename(f)} is stale")
            return None
        total += t["hbm_bytes_per_launch"]
    return total


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, x, min_seconds=10.0):
    """The CPU oracle on the same workload: whole passes over all T tokens,
    repeated until at least `min_seconds` have elapsed."""
    import oracle
    T = x.shape[0]
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.layer(x, w)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": passes * T / dt, "unit": "tokens/s", "cores": oracle.max_threads(),
            "cpu_model": cpu_model(),
            "kind": "oracle", "sample": f"{passes} full pass(es) over the {T} tokens of the same "
            f"workload (router, top-8, 8 routed + shared SwiGLU experts, fp64 accumulation), "
            f"{dt:.1f} s wall"}


def measure_ceilings(read_bytes=2 << 30, mfma_iters=1000, reps=5):
    """Achievable HBM read bandwidth and bf16 MFMA rate on this device, from the
    library's measurement kernels (a streaming read of a buffer 8x the 256 MB
    last-level cache; independent 16x16x32 bf16 MFMA chains), best of `reps`.
    The MFMA loop runs twice: on random operands (what the layer's matrix
    cores see, the ceiling the fractions are stated against) and on nearly
    constant ones; each run also reports the shader clock it sustained
    (s_memtime ticks over s_memrealtime's 100 MHz, summed over the blocks)."""
    import torch
    from int4_grouped_gemm_router_amd import binding as B
    buf = torch.empty(read_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2 * B.CEILING_MFMA_BLOCKS, dtype=torch.int64, device="cuda")

    def best(fn):
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    t_read = best(lambda: B.moe_ceiling_read(buf, sink))
    out = {"hbm_read_gbs": read_bytes / t_read / 1e9, "read_bytes": read_bytes}
    for random, key in ((True, "mfma_bf16"), (False, "mfma_bf16_constant_operands")):
        flops = [0.0]

        def mfma():
            flops[0] = B.moe_ceiling_mfma(mfma_iters, sink, random=random, clocks=clocks)

        t = best(mfma)
        out[key + "_tflops"] = flops[0] / t / 1e12
        out[key + "_clock_mhz"] = B.ceiling_clock_mhz(clocks)
    out["mfma_flops"] = flops[0]
    out["method"] = ("moe_ceiling_read / moe_ceiling_mfma, best of %d event-timed launches; "
                     "mfma_bf16 on random operands" % reps)
    del buf
    return out


def measured_traffic(workload):
    """HBM bytes per gate/up launch from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when it is missing, for another workload, or taken from
    different kernel sources."""
    from int4_grouped_gemm_router_amd import profiling
    if workload != "prefill_t512" or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("sources_sha256") != profiling.sources_digest():
        log("traffic summary is stale (kernel sources changed since the counters were taken)")
        return None
    return t["hbm_bytes_per_launch"]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill_t512")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated (cache guard)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--block-m", type=int, default=32, choices=(16, 32),
                    help="routing block size = GEMM work-item rows (ablation; 32 by default)")
    ap.add_argument("--gemm", default="auto", choices=("auto", "exact", "wide"),
                    help="grouped GEMM design (ablations; the automatic choice by default)")
    ap.add_argument("--unfused", action="store_true",
                    help="ablation: time moe_prefill_layer_unfused against the fused call")
    ap.add_argument("--host-routing", action="store_true",
                    help="ablation: time moe_prefill_layer_host_routed against the GPU-routed call")
    ap.add_argument("--sweep-chunks", action="store_true",
                    help="time the 16384-token prompt at several chunk sizes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from int4_grouped_gemm_router_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from int4_grouped_gemm_router_amd import build as Bd
        Bd.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"device: {torch.cuda.get_device_name(0)}")

    if args.unfused:
        from int4_grouped_gemm_router_amd import binding as B
        rows = []
        for name in ("prefill_t512", "skew_t2048"):
            r, _ = run_prefill(name, args.steps, args.warmup, args.copies,
                               gemm={"auto": 0, "exact": 1, "wide": 2}[args.gemm])
            wl, w, x, xd, dws = prefill_setup(name, args.copies)
            d = dws[0].dims
            T = wl.T
            y = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
            ws = B.workspace(d, T, B.MODE_PREFILL)
            wbuf = B.unfused_weights(d)
            for i in range(args.warmup):
                B.moe_prefill_layer_unfused(d, dws[i % args.copies], xd, y, T, wbuf, ws=ws)
            graphs = [_graph_of(lambda i=i: B.moe_prefill_layer_unfused(d, dws[i], xd, y, T, wbuf, ws=ws))
                      for i in range(args.copies)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                graphs[i % args.copies].replay()
            torch.cuda.synchronize()
            ms_unf = (time.perf_counter() - t0) * 1e3 / args.steps
            row = {"workload": name, "T": T, "ms_fused": r["ms_per_step"], "ms_unfused": ms_unf,
                   "speedup_fused": ms_unf / r["ms_per_step"], "bf16_weight_buffer_bytes": wbuf.numel()}
            log(f"unfused {name}: {row}")
            rows.append(row)
        print(json.dumps({"metric": METRIC, "ablation": "fused vs unfused dequant", "rows": rows}),
              flush=True)
        return
    if args.host_routing:
        from int4_grouped_gemm_router_amd import binding as B
        rows = []
        for name in ("prefill_t512", "skew_t2048"):
            r, _ = run_prefill(name, args.steps, args.warmup, args.copies,
                               gemm={"auto": 0, "exact": 1, "wide": 2}[args.gemm])
            wl, w, x, xd, dws = prefill_setup(name, args.copies)
            d = dws[0].dims
            T = wl.T
            y = torch.empty((T, w.H), dtype=torch.int16, device="cuda")
            ws = B.workspace(d, T, B.MODE_PREFILL)
            for i in range(args.warmup):
                B.moe_prefill_layer_host_routed(d, dws[i % args.copies], xd, y, T, 0, ws)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.steps):
                B.moe_prefill_layer_host_routed(d, dws[i % args.copies], xd, y, T, 0, ws)
            torch.cuda.synchronize()
            ms_host = (time.perf_counter() - t0) * 1e3 / args.steps
            row = {"workload": name, "T": T, "ms_gpu_routed_graph": r["ms_per_step"],
                   "ms_gpu_routed_eager": r["ms_per_step_eager"], "ms_host_routed": ms_host,
                   "speedup_gpu_routed_eager": ms_host / r["ms_per_step_eager"],
                   "speedup_gpu_routed_graph": ms_host / r["ms_per_step"]}
            log(f"host routing {name}: {row}")
            rows.append(row)
        print(json.dumps({"metric": METRIC, "ablation": "host-synchronised routing", "rows": rows}),
              flush=True)
        return
    if args.sweep_chunks:
        from int4_grouped_gemm_router_amd import binding as B
        sweep = []
        for c in (1024, 2048, 4096, 8192, 16384):
            r, (w, _) = run_prefill("long_t16384", 10, 2, args.copies, chunk=c)
            ws_bytes = B.moe_workspace_bytes(B.MoeDims(w.H, w.I, w.E, 8, 32), c, B.MODE_PREFILL)
            row = {"chunk": c, "ms_per_step": r["ms_per_step"], "tokens_per_s": r["tokens_per_s"],
                   "expert_tflops": r["expert_tflops"], "workspace_bytes": ws_bytes,
                   "kernels_us_per_chunk": r["kernels_us"]}
            log(f"chunk {c}: {row}")
            sweep.append(row)
        print(json.dumps({"metric": METRIC, "workload": "long_t16384", "unit": "tokens/s",
                          "sweep": sweep}), flush=True)
        return
    if args.workload.startswith("decode"):
        # decode alone (for profiling): the GEMV bandwidth line of that workload
        r = run_decode(args.workload, args.decode_steps, 20, 32)
        log(f"{args.workload}: {r}")
        print(json.dumps({"metric": METRIC, "value": r["gemv_gbs"], "unit": "GB/s", "n_gpus": 1,
                          "steps": r["steps"], "warmup": 20, "ms_per_step": r["ms_per_step"],
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                          "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": args.workload, "T": r["T"]}, "decode": r}), flush=True)
        return
    gemm = {"auto": 0, "exact": 1, "wide": 2}[args.gemm]
    res, (w, x) = run_prefill(args.workload, args.steps, args.warmup, args.copies,
                              block_m=args.block_m, gemm=gemm)
    log(f"{args.workload}: {res}")
    gu_us = res["kernels_us"]["gemm_gateup"]
    dominant = max(res["kernels_us"], key=res["kernels_us"].get)
    # bound of the gate/up kernel from its arithmetic intensity vs the ridge point
    gu_flops = 2.0 * (8 + 1) * res["T"] * w.H * 2 * w.I
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if "gateup_algorithmic_bytes" in res and gu_flops / res["gateup_algorithmic_bytes"] < ridge:
        roofline = {"bound": "hbm", "achieved": res["gateup_gbs"], "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": res["gateup_gbs"] / PEAK_HBM_GBS,
                    "traffic": measured_traffic(args.workload),
                    "kernel": "gemm_gateup", "per_launch_bytes": res["gateup_algorithmic_bytes"],
                    "mean_us": gu_us}
    else:
        roofline = {"bound": "mfma", "achieved": res["gateup_tflops"], "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": res["gateup_tflops"] / PEAK_BF16_TFLOPS,
                    "traffic": None, "kernel": "gemm_gateup", "mean_us": gu_us}
    roofline["dominant_kernel"] = dominant
    ceil = measure_ceilings()
    log(f"measured ceilings: {ceil}")
    roofline["measured_peak"] = (ceil["hbm_read_gbs"] if roofline["unit"] == "GB/s"
                                 else ceil["mfma_bf16_tflops"])
    roofline["frac_of_measured"] = roofline["achieved"] / roofline["measured_peak"]
    out = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "T": res["T"], "H": w.H, "I": w.I, "E": w.E,
                   "top_k": 8, "shared_experts": 1,
                   "weights": "int4 affine, groups of 64, bf16 scale+bias",
                   "weight_copies": args.copies, "launch": "hip graph per layer call",
                   "block_m": args.block_m, "gemm": args.gemm,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "ceilings": ceil,
        "kernels_us": res["kernels_us"],
        "expert_tflops": res["expert_tflops"],
        "mfma_frac_layer": res["mfma_frac_layer"],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
        log(f"cpu baseline: {out['cpu_baseline']}")
    if not args.no_secondary:
        sec = []
        r2, _ = run_prefill("skew_t2048", max(10, args.steps // 2), args.warmup, args.copies)
        log(f"skew_t2048: {r2}")
        sec.append(r2)
        r4, _ = run_prefill("long_t16384", 10, 2, args.copies)
        log(f"long_t16384: {r4}")
        sec.append(r4)
        r3 = run_decode("decode_t1", args.decode_steps, 20, 32)
        log(f"decode_t1: {r3}")
        sec.append(r3)
        r5 = run_decode("decode_t4", args.decode_steps, 20, 32)
        log(f"decode_t4: {r5}")
        sec.append(r5)
        for r in sec:
            if "expert_tflops" in r:
                r["mfma_frac_of_measured"] = r["expert_tflops"] / ceil["mfma_bf16_tflops"]
            if "gemv_gbs" in r:
                r["hbm_frac_of_measured"] = r["gemv_gbs"] / ceil["hbm_read_gbs"]
        out["secondary"] = sec
        # matrix-core rooflines of the long-chunk configurations (the bf16
        # peak-fraction half of the metric), beside the HBM one above
        out["roofline_mfma"] = {r["workload"]: {"gate_up": r["roofline_gateup"], "down": r["roofline_down"],
                                                "layer_frac": r["mfma_frac_layer"]}
                                for r in (r2, r4)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
