#!/usr/bin/env python3
"""Benchmark: same-device ReduceScatter -> AllGather (Partial -> Shard(0) ->
Replicate, i.e. an AllReduce) of P=8 bf16 [8192, 8192] rank tensors drawn
N(0,1) on one MI355X, with fp32 accumulation in fixed rank order.

One step = dt_reduce_scatter over the 8 rank inputs + dt_all_gather of the
8 shards back into 8 full outputs.  The headline value is the AllReduce bus
bandwidth of that step: algbw = S / t with S = 128 MiB per rank, busbw =
algbw * 2(P-1)/P (the ring-AllReduce volume factor of the c10d page,
sec. 6.1).  Every kernel launch of the timed region is bracketed by HIP
events on the stream it runs on; the dominant kernel's algorithmic HBM bytes
per launch over its mean duration give the roofline fraction against the
MI355X's 8 TB/s.  The CPU oracle, timed on a bounded sample of the same
workload on the host, is reported beside it.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--sweep]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
P = 8
SHAPE = (8192, 8192)
METRIC = "AllReduce/ReduceScatter bus GB/s & % of HBM peak on 1 MI355X, P=8"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("collective_communication_primitives_amd/csrc/reduce.hip",
                  "collective_communication_primitives_amd/csrc/copy.hip",
                  "collective_communication_primitives_amd/csrc/dt_device.h",
                  "collective_communication_primitives_amd/csrc/dt_launch.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"^source_hash:\s*(\S+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def pct(xs, q: float) -> float:
    """q-quantile (0..1) of a sample by linear interpolation."""
    xs = sorted(xs)
    i = q * (len(xs) - 1)
    lo = int(i)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)


def kernel_stats(us, alg_bytes, s_bytes, bus_factor):
    """Per-launch durations (us) -> mean / median / p10 / p90 and rates."""
    mean = statistics.mean(us)
    return {"mean_us": round(mean, 3), "median_us": round(statistics.median(us), 3),
            "p10_us": round(pct(us, 0.1), 3), "p90_us": round(pct(us, 0.9), 3), "alg_bytes": int(alg_bytes),
            "hbm_GBps": round(alg_bytes / (mean * 1e-6) / 1e9, 1),
            "busbw_GBps": round(s_bytes / (mean * 1e-6) / 1e9 * bus_factor, 1)}


def copy_ceiling(torch, stream, steps: int = 10) -> dict:
    """Context for the roofline: torch's own device-to-device copy of 1 GiB
    (read 1 GiB + write 1 GiB), timed per launch like the collectives."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    evs = time_launches(lambda: dst.copy_(src), steps, stream)
    torch.cuda.synchronize()
    us = statistics.mean(a.elapsed_time(b) for a, b in evs) * 1e3
    return {"bytes": 2 << 30, "mean_us": round(us, 3), "hbm_GBps": round((2 << 30) / (us * 1e-6) / 1e9, 1)}


def int32_max_step(dt, torch, steps: int, warmup: int, stream) -> dict:
    """The int32 variant of the same workload: P=8 [8192, 8192] int32 over
    the whole int32 range, max op: ReduceScatter, AllGather and AllReduce,
    each timed per call (at 256 MiB per rank the AllReduce is itself a
    ReduceScatter into each output's own chunk plus an in-place AllGather)."""
    import synth
    n = SHAPE[0] * SHAPE[1]
    xs = synth.full_range_int_ranks(P, n, seed=0, device="cuda")
    shards = [torch.empty(n // P, dtype=torch.int32, device="cuda") for _ in range(P)]
    full = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(P)]
    s_bytes = n * 4
    for _ in range(warmup):
        dt.dt_reduce_scatter(xs, shards, op="max")
        dt.dt_all_gather(shards, full)
    ev_rs, ev_ag = [], []
    for _ in range(steps):
        ev_rs += time_launches(lambda: dt.dt_reduce_scatter(xs, shards, op="max"), 1, stream)
        ev_ag += time_launches(lambda: dt.dt_all_gather(shards, full), 1, stream)
    ev_ar = time_launches(lambda: dt.dt_allreduce(xs, full, op="max"), steps, stream)
    torch.cuda.synchronize()
    us = lambda evs: [a.elapsed_time(b) * 1e3 for a, b in evs]  # noqa: E731
    out = {"reduce_scatter": kernel_stats(us(ev_rs), (P + 1) * s_bytes, s_bytes, (P - 1) / P),
           "all_gather": kernel_stats(us(ev_ag), (1 + P) * s_bytes, s_bytes, (P - 1) / P),
           "allreduce": kernel_stats(us(ev_ar), 2 * P * s_bytes, s_bytes, 2 * (P - 1) / P)}
    step_us = out["reduce_scatter"]["mean_us"] + out["all_gather"]["mean_us"]
    out["step_busbw_GBps"] = round(s_bytes / (step_us * 1e-6) / 1e9 * 2 * (P - 1) / P, 1)
    return out


def time_launches(fn, steps, stream):
    """Run fn() `steps` times with start/end events on `stream` around each."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    return evs


def cpu_baseline(xs_dev, reps: int):
    """The oracle, untouched, timed on the host: RS then AG on the full
    workload copied back from the device, median of `reps` repetitions, each
    timed on its own.  Two legs of the same source: the plain single-threaded
    build, and its OpenMP build over all host cores (every element still
    folded by one thread in rank order: the same bytes).  `value` is the
    all-cores leg; `single_thread` the other."""
    import numpy as np
    import oracle
    host = [x.view(__import__("torch").int16).cpu().numpy().view(np.uint16).reshape(-1) for x in xs_dev]
    s_bytes = host[0].nbytes

    def leg(orc, n):
        times = []
        for _ in range(n):
            t0 = time.perf_counter()
            shards = orc.reduce_scatter(host, "sum")
            orc.all_gather(shards)
            times.append(time.perf_counter() - t0)
        t = statistics.median(times)
        return t, s_bytes / t * 2 * (P - 1) / P / 1e9

    t1, bw1 = leg(oracle.get(), reps)
    omp = oracle.get_omp()
    tn, bwn = leg(omp, max(reps, 25))
    return {"value": round(bwn, 3), "unit": "GB/s", "cores": omp.threads(), "kind": "oracle",
            "sample": f"full workload (P=8 bf16 {SHAPE[0]}x{SHAPE[1]} per rank), RS then AG, median of "
                      f"{max(reps, 25)} runs of {tn:.3f} s on {omp.threads()} OpenMP threads (the oracle's loops "
                      f"built with -fopenmp, same bytes); same busbw formula",
            "seconds_per_step": round(tn, 4),
            "single_thread": {"value": round(bw1, 3), "unit": "GB/s", "cores": 1, "seconds_per_step": round(t1, 3),
                              "sample": f"the same workload, median of {reps} single-threaded runs"},
            "host_cpus": os.cpu_count(), "host_cpu_model": host_cpu_model()}


def host_cpu_model() -> str:
    """The host CPU's model name, as /proc/cpuinfo reports it (empty if unknown)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def graph_time_us(torch, fn, per_graph: int = 20, replays: int = 5) -> float:
    """GPU time per call of fn(): per_graph calls captured in one HIP graph,
    replayed `replays` times back to back; host enqueue cost is excluded."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm the launch path outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (per_graph * replays)


def sweep(dt, torch, steps: int, warmup: int):
    """fp32 AllReduce, P=16, per-rank sizes 4 KiB .. 1 GiB (x4).
    Each point is timed three ways: eager launches bracketed by events (what a
    Python caller sees, host enqueue included), a loop of one prepared call
    (marshalled once) between two events, and graph replay (GPU time per
    launch).  The alpha-beta fit T(S) = alpha + 2*P*S / B_eff (weights 1/T^2)
    uses the graph times."""
    import numpy as np
    import synth
    rows = []
    p = 16
    for nbytes in synth.SWEEP_BYTES:
        n = nbytes // 4
        xs = synth.uniform_ranks(p, n, seed=0, device="cuda")
        ys = [torch.empty_like(x) for x in xs]
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            dt.dt_allreduce(xs, ys)
        evs = time_launches(lambda: dt.dt_allreduce(xs, ys), steps, stream)
        torch.cuda.synchronize()
        eager_us = statistics.median(a.elapsed_time(b) for a, b in evs) * 1e3
        prepared = dt.prepare(dt.dt_allreduce, xs, ys)   # marshalled once: the loop pays the C call only
        a0, b0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(steps):
            prepared()
        b0.record(stream)
        torch.cuda.synchronize()
        prepared_us = a0.elapsed_time(b0) / steps * 1e3
        del prepared
        per_graph = 20 if nbytes <= (16 << 20) else 4
        us = graph_time_us(torch, lambda: dt.dt_allreduce(xs, ys), per_graph=per_graph, replays=5)
        hbm = 2 * p * nbytes / (us * 1e-6) / 1e9
        busbw = nbytes / (us * 1e-6) * 2 * (p - 1) / p / 1e9
        rows.append({"bytes_per_rank": nbytes, "us": round(us, 3), "eager_us": round(eager_us, 3),
                     "prepared_loop_us": round(prepared_us, 3),
                     "hbm_GBps": round(hbm, 1), "busbw_GBps": round(busbw, 1),
                     "frac_of_peak": round(hbm / HBM_PEAK_GBPS, 4)})
        print(json.dumps({"sweep": rows[-1]}), flush=True)
        del xs, ys
        torch.cuda.empty_cache()
    fit = alpha_beta_fit([r["bytes_per_rank"] for r in rows], [r["us"] for r in rows], p)
    print(json.dumps({"sweep_fit": fit}), flush=True)
    return rows, fit


MALL_BYTES = 256 * 1000 ** 2  # the Infinity Cache: 256 MB


def alpha_beta_fit(sizes, us, p: int) -> dict:
    """The single-device alpha-beta model T(S) = alpha + 2*P*S / B (the c10d
    page's sec. 6.1 accounting; alpha dominates small messages, sec. 6.5),
    fitted per regime from graph-replay times:
      alpha: the mean time of the latency points (S <= 64 KiB per rank);
      B_hbm: from the points whose footprint 2*P*S exceeds 512 MiB (twice the
        Infinity Cache), T - alpha weighted 1/T^2;
      B_cache: the same over the points whose footprint fits the Infinity
        Cache and whose time is at least 2 * alpha (below that, T - alpha is
        mostly noise).
    B takes alpha off each point's time (the model), so it can sit a little
    above the best measured rate (by about alpha / T); B_GBps_without_alpha
    is the same weighted mean of the measured rates themselves."""
    s = [float(x) for x in sizes]
    t = [float(x) * 1e-6 for x in us]
    lat = [ti for si, ti in zip(s, t) if si <= 64 * 1024]
    alpha = statistics.mean(lat) if lat else 0.0

    def band(sel):
        pts = [(2 * p * si, ti) for si, ti in zip(s, t) if sel(si, ti)]
        if not pts:
            return None
        num = sum(x * x / (ti * ti) for x, ti in pts)
        den = sum(x * (ti - alpha) / (ti * ti) for x, ti in pts)
        rates = [x / ti for x, ti in pts]
        return {"B_GBps": round(num / den / 1e9, 1) if den > 0 else None, "points": len(pts),
                "best_point_GBps": round(max(rates) / 1e9, 1),
                # the same weights without the alpha correction: a weighted mean of
                # the measured rates, so never above the best point
                "B_GBps_without_alpha": round(sum(r * r for r in rates) / sum(rates) / 1e9, 1)}

    return {"alpha_us": round(alpha * 1e6, 3),
            "hbm": band(lambda si, ti: 2 * p * si > 512 * 2 ** 20),
            "cache": band(lambda si, ti: 2 * p * si <= MALL_BYTES and si > 64 * 1024 and ti >= 2 * alpha),
            "model": "T(S) = alpha + 2*P*S/B, P=16, graph-replay times; alpha from S <= 64 KiB, B per regime "
                     "(weights 1/T^2): hbm = footprint > 512 MiB, cache = footprint within the 256 MB Infinity Cache "
                     "and T >= 2 alpha"}


def hsdp(dt, torch):
    """The gradient workload: P=8, 32 layers x 9 bf16 tensors per rank
    (103.6 GB), 25 MiB buckets.
      replicate2_shard4: the per-layer ReduceScatter -> fused AllReduce
        pipeline (time from the first post_backward to the consumer's wait),
        one stream per phase, the same with one side stream for both, and
        with both on the stream that produced the gradients;
      ddp_bucket: pure data parallel, each layer's tensors AllReduced in
        place in 25 MiB buckets (dt_bucket_allreduce, no staging copies)."""
    import numpy as np
    import synth
    out = {}
    layers = [synth.layer_grads(P, layer=l, seed=0, device="cuda") for l in range(synth.NUM_LAYERS)]
    numels = [int(np.prod(s)) for s in synth.LAYER_SHAPES]
    per_rank_layer = sum(numels) * 2

    def timed(run, reps=3):
        times = []
        for it in range(reps + 1):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            a.record()
            run()
            b.record()
            host_ms = (time.perf_counter() - t0) * 1e3
            torch.cuda.synchronize()
            if it > 0:  # the first pass warms up
                times.append((a.elapsed_time(b), host_ms))
        return statistics.median(t for t, _ in times), statistics.median(h for _, h in times)

    rep, sh = 2, 4
    fused = [[torch.empty(sum(numels) // sh, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
             for _ in range(synth.NUM_LAYERS)]
    pipe = dt.HSDPPipeline(rep, sh, bucket_bytes=synth.BUCKET_BYTES, rs_stream=torch.cuda.Stream(),
                           ar_stream=torch.cuda.Stream())

    def run_hsdp():
        for l in reversed(range(synth.NUM_LAYERS)):
            pipe.post_backward(layers[l], fused[l])
        pipe.finish()

    ms, host_ms = timed(run_hsdp)
    # ReduceScatter: per shard group, shard reads + 1 write of one rank's layer
    # bytes; fused AllReduce: read + write of every rank's fused buffer
    total = synth.NUM_LAYERS * (rep * (sh + 1) * per_rank_layer + 2 * P * (per_rank_layer // sh))
    out["replicate2_shard4"] = {"ms": round(ms, 3), "host_enqueue_ms": round(host_ms, 3), "alg_bytes": total,
                                "hbm_GBps": round(total / (ms * 1e-3) / 1e9, 1),
                                "frac_of_peak": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    print(json.dumps({"hsdp": out}), flush=True)
    del pipe

    # the same pipeline with one stream for both phases: on one device the
    # ReduceScatter and the AllReduce compete for the same HBM, so running them
    # back to back (in the same issue order) is the other schedule to measure
    pipe = dt.HSDPPipeline(rep, sh, bucket_bytes=synth.BUCKET_BYTES)  # default: one side stream
    ms, host_ms = timed(run_hsdp)
    out["replicate2_shard4_one_stream"] = {"ms": round(ms, 3), "host_enqueue_ms": round(host_ms, 3),
                                           "alg_bytes": total, "hbm_GBps": round(total / (ms * 1e-3) / 1e9, 1),
                                           "frac_of_peak": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    print(json.dumps({"hsdp": out}), flush=True)
    del pipe
    # both phases on the stream that produced the gradients (here torch's
    # current stream): the pipeline then needs no cross-stream events
    cur = torch.cuda.current_stream()
    pipe = dt.HSDPPipeline(rep, sh, bucket_bytes=synth.BUCKET_BYTES, rs_stream=cur, ar_stream=cur)
    ms, host_ms = timed(run_hsdp)
    out["replicate2_shard4_producer_stream"] = {"ms": round(ms, 3), "host_enqueue_ms": round(host_ms, 3),
                                                "alg_bytes": total, "hbm_GBps": round(total / (ms * 1e-3) / 1e9, 1),
                                                "frac_of_peak": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    print(json.dumps({"hsdp": out}), flush=True)
    del fused, pipe
    torch.cuda.empty_cache()

    def run_ddp():
        for l in reversed(range(synth.NUM_LAYERS)):
            dt.dt_bucket_allreduce(layers[l], bucket_bytes=synth.BUCKET_BYTES)

    ms, host_ms = timed(run_ddp)
    total = synth.NUM_LAYERS * 2 * P * per_rank_layer
    out["ddp_bucket"] = {"ms": round(ms, 3), "host_enqueue_ms": round(host_ms, 3), "alg_bytes": total,
                         "hbm_GBps": round(total / (ms * 1e-3) / 1e9, 1),
                         "frac_of_peak": round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    print(json.dumps({"hsdp": out}), flush=True)
    del layers
    torch.cuda.empty_cache()
    return out


def frac_of_peak(alg_bytes: float, us: float) -> float:
    return round(alg_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)


def configs(dt, torch, steps: int, warmup: int) -> dict:
    """One timing of each workload besides the bench step, in bounded time:
      c1_allreduce_p4: P=4, 1,048,576 fp32 and int32 elements per rank
        (cache-resident, latency-bound: graph-replay us per call);
      c3_uneven_all_gather_p8 / c3_all_to_all_p8: fp32 rows of 4096, row
        counts U[1, 16384] / a U[0, 4096]-row split matrix;
      c5_allreduce_p16: the sweep's HBM-resident points, fp32 16 MiB .. 1 GiB
        per rank (graph replay);
      c5_barrier_p16: 1000 generations of the packed barrier in one launch;
      c4_pipeline_pass: one pass of the 32-layer gradient pipeline (replicate
        2 x shard 4, one stream, 25 MiB buckets).
    Every entry carries its algorithmic HBM bytes and fraction of peak."""
    import numpy as np
    import synth
    stream = torch.cuda.current_stream()
    out = {}

    def measure(name, fn, alg_bytes, per_graph=10, replays=3, events=True):
        for _ in range(warmup):
            fn()
        row = {"alg_bytes": int(alg_bytes)}
        if events:
            evs = time_launches(fn, steps, stream)
            torch.cuda.synchronize()
            us = statistics.mean(a.elapsed_time(b) for a, b in evs) * 1e3
            row["mean_us"] = round(us, 3)
        g = graph_time_us(torch, fn, per_graph=per_graph, replays=replays)
        row["graph_us"] = round(g, 3)
        row["frac_of_peak"] = frac_of_peak(alg_bytes, row.get("mean_us", g))
        row["frac_of_peak_graph"] = frac_of_peak(alg_bytes, g)
        out[name] = row
        print(json.dumps({name: row}), flush=True)

    n = 1 << 20
    for dtype, xs in (("fp32", synth.uniform_ranks(4, n, seed=0, device="cuda")),
                      ("int32", synth.int_ranks(4, n, seed=0, device="cuda"))):
        ys = [torch.empty_like(x) for x in xs]
        measure(f"c1_allreduce_p4_{dtype}", lambda: dt.dt_allreduce(xs, ys), 2 * 4 * n * 4, per_graph=20, replays=5)
        out[f"c1_allreduce_p4_{dtype}"]["note"] = "32 MiB footprint: cache-resident, latency-bound"
        del xs, ys

    w = synth.ROW_WIDTH
    counts = synth.uneven_row_counts(seed=0)
    xs = synth.uniform_rows(counts, w, seed=100, device="cuda")
    total = int(counts.sum()) * w
    ys = [torch.empty(total, device="cuda") for _ in range(P)]
    measure("c3_uneven_all_gather_p8", lambda: dt.dt_all_gather(xs, ys), (1 + P) * total * 4, per_graph=4)
    del xs, ys
    s_rows = synth.split_matrix(seed=0)
    xs = synth.uniform_rows([int(s_rows[i].sum()) for i in range(P)], w, seed=200, device="cuda")
    ys = [torch.empty(int(s_rows[:, j].sum()) * w, device="cuda") for j in range(P)]
    measure("c3_all_to_all_p8", lambda: dt.dt_all_to_all(xs, ys, (s_rows * w).tolist()),
            2 * int(s_rows.sum()) * w * 4, per_graph=4)
    del xs, ys
    torch.cuda.empty_cache()

    # misaligned buffers: the step's AllReduce on views 2 bytes past 16-byte
    # alignment (every buffer off by the same amount), and the uneven
    # AllGather in bf16 with odd counts (every later piece lands 2 bytes off)
    n = SHAPE[0] * SHAPE[1]
    base = [torch.randn(n + 8, device="cuda").to(torch.bfloat16) for _ in range(P)]
    outb = [torch.empty(n + 8, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    xs, ys = [b[1:1 + n] for b in base], [b[1:1 + n] for b in outb]
    measure("c2_allreduce_misaligned_p8_bf16", lambda: dt.dt_allreduce(xs, ys), 2 * P * n * 2, per_graph=4)
    out["c2_allreduce_misaligned_p8_bf16"]["note"] = "every buffer 2 bytes past 16-byte alignment"
    xs = [b[:n] for b in base]
    measure("c2_allreduce_outputs_misaligned_p8_bf16", lambda: dt.dt_allreduce(xs, ys), 2 * P * n * 2, per_graph=4)
    out["c2_allreduce_outputs_misaligned_p8_bf16"]["note"] = \
        "inputs aligned, outputs 2 bytes past 16-byte alignment: the line-grid two-shot form"
    ro = [torch.empty(n // P + 8, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    rs_out = [r[1:n // P + 1] for r in ro]
    measure("c2_reduce_scatter_outputs_misaligned_p8_bf16", lambda: dt.dt_reduce_scatter(xs, rs_out),
            (P + 1) * n * 2, per_graph=4)
    out["c2_reduce_scatter_outputs_misaligned_p8_bf16"]["note"] = \
        "inputs aligned, outputs 2 bytes past 16-byte alignment: offsets that no peel can share"
    del base, outb, xs, ys, ro, rs_out
    rows_odd = [int(c) * w + 2 * k + 1 for k, c in enumerate(counts)]
    xs = [torch.randn(c, device="cuda").to(torch.bfloat16) for c in rows_odd]
    ys = [torch.empty(sum(rows_odd), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    measure("c3_uneven_all_gather_odd_bf16", lambda: dt.dt_all_gather(xs, ys), (1 + P) * sum(rows_odd) * 2,
            per_graph=4)
    out["c3_uneven_all_gather_odd_bf16"]["note"] = "bf16, odd counts: every piece after the first 2 bytes off"
    del xs, ys
    torch.cuda.empty_cache()

    rows = []
    for nbytes in (16 << 20, 64 << 20, 256 << 20, 1 << 30):
        xs = synth.uniform_ranks(16, nbytes // 4, seed=0, device="cuda")
        ys = [torch.empty_like(x) for x in xs]
        for _ in range(2):
            dt.dt_allreduce(xs, ys)
        g = graph_time_us(torch, lambda: dt.dt_allreduce(xs, ys), per_graph=2 if nbytes >= (256 << 20) else 4,
                          replays=4)
        alg = 2 * 16 * nbytes
        rows.append({"bytes_per_rank": nbytes, "graph_us": round(g, 3), "alg_bytes": alg,
                     "frac_of_peak": frac_of_peak(alg, g),
                     "busbw_GBps": round(nbytes / (g * 1e-6) * 2 * 15 / 16 / 1e9, 1)})
        print(json.dumps({"c5_allreduce_p16": rows[-1]}), flush=True)
        del xs, ys
        torch.cuda.empty_cache()
    out["c5_allreduce_p16_fp32"] = rows

    ws = [torch.zeros(16, dtype=torch.int32, device="cuda") for _ in range(16)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dt.dt_barrier(ws, status, 1, 10)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    dt.dt_barrier(ws, status, 11, 1000)
    b.record()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    out["c5_barrier_p16"] = {"us_per_generation": round(a.elapsed_time(b) * 1e3 / 1000, 3), "generations": 1000,
                             "layout": "packed", "alg_bytes": 0}
    print(json.dumps({"c5_barrier_p16": out["c5_barrier_p16"]}), flush=True)

    layers = [synth.layer_grads(P, layer=l, seed=0, device="cuda") for l in range(synth.NUM_LAYERS)]
    numels = [int(np.prod(sh)) for sh in synth.LAYER_SHAPES]
    per_rank_layer = sum(numels) * 2
    rep, sh = 2, 4
    fused = [[torch.empty(sum(numels) // sh, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
             for _ in range(synth.NUM_LAYERS)]
    pipe = dt.HSDPPipeline(rep, sh, bucket_bytes=synth.BUCKET_BYTES)
    times = []
    for it in range(3):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for l in reversed(range(synth.NUM_LAYERS)):
            pipe.post_backward(layers[l], fused[l])
        pipe.finish()
        b.record()
        torch.cuda.synchronize()
        if it > 0:  # the first pass warms up
            times.append(a.elapsed_time(b))
    alg = synth.NUM_LAYERS * (rep * (sh + 1) * per_rank_layer + 2 * P * (per_rank_layer // sh))
    ms = statistics.median(times)
    out["c4_pipeline_pass"] = {"ms": round(ms, 3), "alg_bytes": alg, "frac_of_peak": frac_of_peak(alg, ms * 1e3),
                               "mesh": "replicate 2 x shard 4, one stream", "passes_timed": len(times)}
    print(json.dumps({"c4_pipeline_pass": out["c4_pipeline_pass"]}), flush=True)
    pipe.close()
    del layers, fused, pipe
    torch.cuda.empty_cache()
    return out


def barrier_latency(dt, torch):
    """P=16 signal-window barrier, both layouts: 1000 generations in one
    launch (us per generation), and 1000 single-generation launches queued
    eagerly from Python (us per launch).  Graph replay cannot time a barrier:
    its thresholds would be frozen into the graph."""
    p = 16
    out = {"P": p}
    for layout in ("packed", "spread"):
        ws = [torch.zeros(p, dtype=torch.int32, device="cuda") for _ in range(p)]
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        dt.dt_barrier(ws, status, 1, 10, layout=layout)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dt.dt_barrier(ws, status, 11, 1000, layout=layout)
        b.record()
        torch.cuda.synchronize()
        in_kernel = a.elapsed_time(b) * 1e3 / 1000
        a.record()
        for g in range(1011, 2011):
            dt.dt_barrier(ws, status, g, 1, layout=layout)
        b.record()
        torch.cuda.synchronize()
        per_launch = a.elapsed_time(b) * 1e3 / 1000
        out[layout] = {"us_per_generation_in_kernel": round(in_kernel, 3), "us_per_launch_eager": round(per_launch, 3)}
        assert int(status.item()) == 0
    print(json.dumps({"barrier": out}), flush=True)
    return out


def other_rows(dt, torch, steps: int, warmup: int):
    """The remaining workloads, each timed per launch (HIP events around every
    launch; mean) against its algorithmic HBM bytes:
      allreduce_p4: fp32 and int32, P=4, 1,048,576 elements per rank
        (32 MiB per launch, within the Infinity Cache: latency-bound);
      uneven_all_gather_p8: fp32 rows of 4096, row counts U[1, 16384];
      all_to_all_p8: fp32 rows of 4096, split matrix U[0, 4096] rows;
      the placement extras at P=8 bf16: AVG AllReduce and ReplicateToShard of
        [8192, 8192] per rank, Broadcast of one such tensor, AllGatherIntoVec
        of 16 MiB shards, and the AllToAll between shard dimensions of a
        [32768, 16384] tensor (1 GiB) in both directions."""
    import numpy as np
    import synth
    stream = torch.cuda.current_stream()
    out = {}

    def measure(name, fn, alg_bytes):
        for _ in range(warmup):
            fn()
        evs = time_launches(fn, steps, stream)
        torch.cuda.synchronize()
        us = statistics.mean(a.elapsed_time(b) for a, b in evs) * 1e3
        graph_us = graph_time_us(torch, fn, per_graph=10, replays=3)
        out[name] = {"mean_us": round(us, 3), "graph_us": round(graph_us, 3), "alg_bytes": int(alg_bytes),
                     "hbm_GBps": round(alg_bytes / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(alg_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}
        print(json.dumps({name: out[name]}), flush=True)

    n = 1 << 20
    for dtype, xs in (("fp32", synth.uniform_ranks(4, n, seed=0, device="cuda")),
                      ("int32", synth.int_ranks(4, n, seed=0, device="cuda"))):
        ys = [torch.empty_like(x) for x in xs]
        measure(f"allreduce_p4_{dtype}", lambda: dt.dt_allreduce(xs, ys), 2 * 4 * n * 4)
        del xs, ys

    w = synth.ROW_WIDTH
    counts = synth.uneven_row_counts(seed=0)
    xs = synth.uniform_rows(counts, w, seed=100, device="cuda")
    total = int(counts.sum()) * w
    ys = [torch.empty(total, device="cuda") for _ in range(P)]
    measure("uneven_all_gather_p8", lambda: dt.dt_all_gather(xs, ys), (1 + P) * total * 4)
    out["uneven_all_gather_p8"]["rows"] = counts.tolist()
    del xs, ys
    torch.cuda.empty_cache()

    # placement-matrix extras, P=8
    xs = synth.normal_ranks(P, SHAPE, seed=0, device="cuda", dtype=torch.bfloat16)
    ys = [torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    s_bytes = SHAPE[0] * SHAPE[1] * 2
    measure("allreduce_avg_p8_bf16", lambda: dt.dt_allreduce(xs, ys, op="avg"), 2 * P * s_bytes)
    shard = [torch.empty(SHAPE[0] * SHAPE[1] // P, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    measure("replicate_to_shard_p8_bf16", lambda: dt.dt_replicate_to_shard(xs, shard), 2 * s_bytes)
    measure("broadcast_p8_bf16", lambda: dt.dt_broadcast(xs[0], ys), (1 + P) * s_bytes)
    vec = [[torch.empty_like(shard[r]) for r in range(P)] for _ in range(P)]
    measure("all_gather_into_vec_p8_bf16", lambda: dt.dt_all_gather_into_vec(shard, vec), (1 + P) * s_bytes)
    del xs, ys, shard, vec
    torch.cuda.empty_cache()
    rows, cols = 32768, 16384  # bf16, 1 GiB in total
    blk = rows * cols // P
    xs = [torch.randn(blk, device="cuda").to(torch.bfloat16) for _ in range(P)]
    ys = [torch.empty(blk, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    measure("all_to_all_dims_0to1_p8_bf16", lambda: dt.dt_all_to_all_dims(xs, ys, rows, cols, 0, 1), 2 * rows * cols * 2)
    measure("all_to_all_dims_1to0_p8_bf16", lambda: dt.dt_all_to_all_dims(xs, ys, rows, cols, 1, 0), 2 * rows * cols * 2)
    del xs, ys
    torch.cuda.empty_cache()

    s_rows = synth.split_matrix(seed=0)
    s_el = (s_rows * w).tolist()
    xs = synth.uniform_rows([int(s_rows[i].sum()) for i in range(P)], w, seed=200, device="cuda")
    ys = [torch.empty(int(s_rows[:, j].sum()) * w, device="cuda") for j in range(P)]
    measure("all_to_all_p8", lambda: dt.dt_all_to_all(xs, ys, s_el), 2 * int(s_rows.sum()) * w * 4)
    out["all_to_all_p8"]["total_rows"] = int(s_rows.sum())
    del xs, ys
    torch.cuda.empty_cache()
    return out


def overlap(dt, torch, reps: int = 40):
    """Compute/communication overlap on one GPU, after the probe of the c10d
    page (sec. 6, sec. 10.4): a bf16 [8192,8192] x [8192,8192] GEMM
    (torch.matmul, a library GEMM) on the compute stream and the fp32 25 MiB
    bucket AllReduce of P=8 ranks on a side stream.  Events on both streams
    put both kernels on one clock; medians over `reps` runs.
      overlap = (t_gemm + t_ar - t_both) / min(t_gemm, t_ar)
    with t_gemm and t_ar each kernel's own duration when it runs alone and
    t_both the span from the first kernel's start to the last one's end
    (1 = the AllReduce fully hidden, 0 = serialized, below 0 = a gap).  Two issue orders, and
    the page's overlap "killers" placed between issuing the AllReduce and the
    GEMM (sec. 6.3): wait() too early, .item() (a device-to-host read on the
    compute stream), torch.cuda.synchronize(), the caching allocator
    returning memory (empty_cache frees a cached block: an implicit device
    synchronization, the page's cudaFree case) and the AllReduce on the
    compute stream itself (async_op=False)."""
    import synth
    xs = synth.uniform_ranks(P, synth.BUCKET_BYTES // 4, seed=0, device="cuda")
    ys = [torch.empty_like(x) for x in xs]
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    # the "previous layer" for the .item() killer: a GEMM still queued on the
    # compute stream when the host reads a scalar it produces (a loss)
    pa = torch.randn(4096, 4096, device="cuda").to(torch.bfloat16)
    comp, side = torch.cuda.current_stream(), dt.side_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def run(order):
        if order == "frag":
            spare = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
            del spare  # back in the caching allocator's free list
        torch.cuda.synchronize()
        t0, s0, s1, g0, g1, t1 = ev(), ev(), ev(), ev(), ev(), ev()
        t0.record(comp)

        def ar(stream=side):
            if stream is not comp:
                stream.wait_stream(comp)
            s0.record(stream)
            dt.dt_allreduce(xs, ys, stream=stream)
            s1.record(stream)

        def gemm():
            g0.record(comp)
            torch.matmul(a, b)
            g1.record(comp)

        if order == "gemm":
            gemm()
        elif order == "ar":
            ar()
        elif order == "ar_first":
            ar()
            gemm()
        elif order == "gemm_first":
            gemm()
            ar()
        elif order == "wait_too_early":
            ar()
            comp.wait_stream(side)
            gemm()
        elif order == "item":
            loss = torch.matmul(pa, pa)[0, 0]  # queued on the compute stream before the AllReduce
            ar()
            loss.item()  # the host waits for that GEMM before it can issue the next one
            gemm()
        elif order == "sync":
            ar()
            torch.cuda.synchronize()
            gemm()
        elif order == "frag":
            ar()
            torch.cuda.empty_cache()  # releases the block freed below: hipFree, a device-wide wait
            gemm()
        elif order == "same_stream":
            ar(stream=comp)
            gemm()
        comp.wait_stream(side)
        t1.record(comp)
        torch.cuda.synchronize()
        out = {"total_ms": t0.elapsed_time(t1)}
        if order != "gemm":
            out["ar_start_ms"], out["ar_end_ms"] = t0.elapsed_time(s0), t0.elapsed_time(s1)
        if order != "ar":
            out["gemm_start_ms"], out["gemm_end_ms"] = t0.elapsed_time(g0), t0.elapsed_time(g1)
        starts = [v for k, v in out.items() if k.endswith("_start_ms")]
        ends = [v for k, v in out.items() if k.endswith("_end_ms")]
        out["span_ms"] = max(ends) - min(starts)
        return out

    killers = ("wait_too_early", "item", "sync", "frag", "same_stream")
    orders = ("gemm", "ar", "ar_first", "gemm_first") + killers
    samples = {o: [] for o in orders}
    for it in range(reps + 2):
        for o in orders:  # interleaved, so clock drift hits every mode alike
            r = run(o)
            if it >= 2:
                samples[o].append(r)
    med = {o: {k: round(statistics.median(r[k] for r in samples[o]), 4) for k in samples[o][0]} for o in orders}
    t_g, t_a = med["gemm"]["span_ms"], med["ar"]["span_ms"]
    out = {"gemm_ms": t_g, "allreduce_ms": t_a, "gemm_tflops": round(2 * 8192 ** 3 / (t_g * 1e-3) / 1e12, 1)}
    for o in ("ar_first", "gemm_first") + killers:
        per = [(t_g + t_a - r["span_ms"]) / min(t_g, t_a) for r in samples[o]]
        out[o] = dict(med[o], overlap=round((t_g + t_a - med[o]["span_ms"]) / min(t_g, t_a), 3),
                      overlap_p25_p75=[round(pct(per, 0.25), 3), round(pct(per, 0.75), 3)])
    print(json.dumps({"overlap": out}), flush=True)
    return out


def coalescing(dt, torch):
    """The three ways of the c10d page (sec. 6.5) to reduce many small
    gradients, P=8, 1000 bf16 tensors of 25 KB per rank (25 MB in all):
      per_tensor   one dt_allreduce per tensor (1000 launches);
      coalesced    dt_allreduce_coalesced: one launch over a table of the
                   non-contiguous tensors (512 per launch);
      bucket_copy  DDP bucket with a staging buffer: flatten -> AllReduce ->
                   unflatten (three multi-tensor launch groups, 3x the bytes);
      bucket_inplace  the same buckets reduced in place (no staging copies).
    Timed eagerly from Python and by graph replay (GPU time)."""
    import synth
    n_t, n_el = 1000, 12800
    grads = [[torch.randn(n_el, device="cuda").to(torch.bfloat16) for _ in range(n_t)] for _ in range(P)]
    ws = [torch.empty(synth.BUCKET_BYTES, dtype=torch.uint8, device="cuda") for _ in range(P)]
    alg = 2 * P * n_t * n_el * 2

    def per_tensor():
        for t in range(n_t):
            dt.dt_allreduce([grads[r][t] for r in range(P)])

    styles = {"per_tensor": per_tensor,
              "coalesced": lambda: dt.dt_allreduce_coalesced(grads),
              "bucket_copy": lambda: dt.dt_bucket_allreduce(grads, synth.BUCKET_BYTES, bucket_ws=ws),
              "bucket_inplace": lambda: dt.dt_bucket_allreduce(grads, synth.BUCKET_BYTES)}
    out = {"tensors": n_t, "bytes_per_tensor": n_el * 2, "ranks": P, "alg_bytes": alg}
    for name, fn in styles.items():
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(3):
            fn()
        b.record()
        torch.cuda.synchronize()
        eager_us = a.elapsed_time(b) * 1e3 / 3
        g_us = graph_time_us(torch, fn, per_graph=1, replays=5)
        out[name] = {"eager_us": round(eager_us, 1), "graph_us": round(g_us, 1),
                     "hbm_GBps_graph": round(alg / (g_us * 1e-6) / 1e9, 1)}
        print(json.dumps({"coalescing": {name: out[name]}}), flush=True)
    del grads, ws
    torch.cuda.empty_cache()
    return out


def probe(dt, torch, reps: int = 10):
    """Workload for hardware-counter passes: the bench kernels and a plain
    copy of known size (1 GiB read + 1 GiB written) to calibrate
    FETCH_SIZE / WRITE_SIZE against known bytes."""
    import synth
    xs = synth.normal_ranks(P, SHAPE, seed=0, device="cuda", dtype=torch.bfloat16)
    n = SHAPE[0] * SHAPE[1]
    shards = [torch.empty(n // P, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    full = [torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        dt.dt_reduce_scatter(xs, shards)
        dt.dt_all_gather(shards, full)
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "done", "reps": reps, "copy_bytes_each_way": a.numel() * 4}), flush=True)


def probe_rows(dt, torch, reps: int = 3):
    """Workload for hardware-counter passes over the other scope rows, each
    call repeated ``reps`` times with a synchronization in between, plus the
    same 1 GiB copy as ``probe`` to calibrate the counters.  The workloads
    run one after another, so a counter CSV splits by dispatch order (the
    uneven AllGather and the two-shot AllReduce share the gather kernel): the
    AllToAll (k_all_to_all), the uneven AllGather (the windowed fan-out and
    its read pass), the two-shot AllReduce at the bench step's shape (its
    ReduceScatter and gather), one layer of the in-place bucket AllReduce
    (two-shot AllReduces of its large tensors, the fold of the small ones at
    P=8), one layer of the gradient pipeline (the segmented ReduceScatter
    at P=4 and the bucket folds at P=2), the AllToAll between shard
    dimensions of the bf16 [32768, 16384] tensor in both directions, the
    ReplicateToShard of [8192, 8192] bf16 per rank, the AllReduce of the
    bench step's inputs 2 bytes off alignment, the ReduceScatter of the same
    inputs into outputs 2 bytes off (the line-grid kernel) and the uneven
    AllGather in bf16 with odd counts.  Prints one JSON line per workload
    with its algorithmic bytes."""
    import numpy as np
    import synth
    w = synth.ROW_WIDTH

    def run(name, fn, alg_bytes, kernels):
        for _ in range(reps):
            fn()
            torch.cuda.synchronize()
        print(json.dumps({"probe_row": name, "reps": reps, "alg_bytes_per_call": int(alg_bytes),
                          "kernels": kernels}), flush=True)
        torch.zeros(1, device="cuda")  # a fill kernel: marks the workload's end in the dispatch order
        torch.cuda.synchronize()

    s_rows = np.random.default_rng(1).integers(0, 4097, (P, P))
    xs = synth.uniform_rows(s_rows.sum(axis=1), w, seed=200, device="cuda")
    ys = [torch.empty(int(s_rows[:, j].sum()) * w, device="cuda") for j in range(P)]
    run("all_to_all_p8", lambda: dt.dt_all_to_all(xs, ys, (s_rows * w).tolist()), 2 * int(s_rows.sum()) * w * 4,
        ["k_all_to_all"])
    del xs, ys
    counts = synth.uneven_row_counts(seed=0)
    xs = synth.uniform_rows(counts, w, seed=100, device="cuda")
    ys = [torch.empty(int(counts.sum()) * w, device="cuda") for _ in range(P)]
    run("uneven_all_gather_p8", lambda: dt.dt_all_gather(xs, ys), (1 + P) * int(counts.sum()) * w * 4,
        ["k_gather<8, true, 1, 128>", "k_gather_touch"])
    del xs, ys
    torch.cuda.empty_cache()
    xs = synth.normal_ranks(P, SHAPE, seed=0, device="cuda", dtype=torch.bfloat16)
    ys = [torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    s_bytes = SHAPE[0] * SHAPE[1] * 2
    run("allreduce_two_shot_p8_bf16", lambda: dt.dt_allreduce(xs, ys), 2 * P * s_bytes,
        ["k_reduce_scatter_vec<1, 0, 8, 64, 1>", "k_gather<8, true, 1, 64>"])
    del xs, ys
    torch.cuda.empty_cache()
    layer = synth.layer_grads(P, layer=0, seed=0, device="cuda")
    numels = [int(np.prod(sh)) for sh in synth.LAYER_SHAPES]
    per_rank_layer = sum(numels) * 2
    run("bucket_allreduce_layer_p8", lambda: dt.dt_bucket_allreduce(layer, bucket_bytes=synth.BUCKET_BYTES),
        2 * P * per_rank_layer, ["k_reduce_scatter_vec<1, 0, 8, 64, 1>", "k_gather<8, true, 1, 64>",
                                 "k_reduce_pieces<dt::PieceArgs, 1, 0, 8>"])
    rep, sh = 2, 4
    fused = [torch.empty(sum(numels) // sh, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    pipe = dt.HSDPPipeline(rep, sh, bucket_bytes=synth.BUCKET_BYTES)

    def one_layer():
        pipe.post_backward(layer, fused)
        pipe.finish()
    run("gradient_pipeline_layer_r2s4", one_layer,
        rep * (sh + 1) * per_rank_layer + 2 * P * (per_rank_layer // sh),
        ["k_reduce_scatter_segs<1, 0, 4, 1>", "k_reduce_pieces<dt::PieceArgs, 1, 0, 2>"])
    del pipe, fused, layer
    torch.cuda.empty_cache()
    rows, cols = 32768, 16384
    blk = rows * cols // P
    xs = [torch.randn(blk, device="cuda").to(torch.bfloat16) for _ in range(P)]
    ys = [torch.empty(blk, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    for sd, dd in ((0, 1), (1, 0)):
        run(f"all_to_all_dims_{sd}to{dd}_p8_bf16", lambda: dt.dt_all_to_all_dims(xs, ys, rows, cols, sd, dd),
            2 * rows * cols * 2, ["k_all_to_all_dims_wave"])
    del xs, ys
    torch.cuda.empty_cache()
    xs = synth.normal_ranks(P, SHAPE, seed=0, device="cuda", dtype=torch.bfloat16)
    shard = [torch.empty(SHAPE[0] * SHAPE[1] // P, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    run("replicate_to_shard_p8_bf16", lambda: dt.dt_replicate_to_shard(xs, shard), 2 * s_bytes, ["k_copy_segments"])
    del shard
    n = SHAPE[0] * SHAPE[1]
    xo = [torch.empty(n + 8, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    yo = [torch.empty(n + 8, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    for x, src in zip(xo, xs):
        x[1:n + 1].copy_(src.reshape(-1))
    run("allreduce_misaligned_p8_bf16", lambda: dt.dt_allreduce([x[1:n + 1] for x in xo], [y[1:n + 1] for y in yo]),
        2 * P * s_bytes, ["k_reduce_elems", "k_reduce_scatter_vec<1, 0, 8, 64, 1>", "k_gather<8, true, 1, 64>"])
    # the ReduceScatter with aligned inputs and outputs 2 bytes off: the line-grid kernel
    ro = [torch.empty(n // P + 8, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    run("reduce_scatter_outputs_off_p8_bf16", lambda: dt.dt_reduce_scatter(xs, [r[1:n // P + 1] for r in ro]),
        (P + 1) * s_bytes, ["k_reduce_scatter_grid<1, 0, 8>"])
    del xs, xo, yo, ro
    torch.cuda.empty_cache()
    # the uneven AllGather in bf16 with odd counts (pieces 2 or 8 bytes off: the line-grid fan-out)
    rows_odd = [int(c) * w + 2 * k + 1 for k, c in enumerate(counts)]
    xs = [torch.randn(c, device="cuda").to(torch.bfloat16) for c in rows_odd]
    ys = [torch.empty(sum(rows_odd), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    run("uneven_all_gather_odd_bf16_p8", lambda: dt.dt_all_gather(xs, ys), (1 + P) * sum(rows_odd) * 2,
        ["k_gather<8, true, 1, 128>", "k_gather_touch"])
    del xs, ys
    torch.cuda.empty_cache()
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "done", "reps": reps, "copy_bytes_each_way": a.numel() * 4}), flush=True)


def probe_sweep(dt, torch, reps: int = 3):
    """Workload for hardware-counter passes over the HBM-resident points of
    the P=16 fp32 AllReduce sweep (16 MiB, 64 MiB, 256 MiB and 1 GiB per
    rank), each call repeated ``reps`` times with a synchronization in
    between, then the 1 GiB copy that calibrates the counters.  Prints one
    JSON line per point with its algorithmic bytes (2 * P * S) and the
    number of kernel dispatches one call makes, so a counter CSV splits by
    dispatch order."""
    import synth
    p = 16
    for nbytes in (16 << 20, 64 << 20, 256 << 20, 1 << 30):
        xs = synth.uniform_ranks(p, nbytes // 4, seed=0, device="cuda")
        ys = [torch.empty_like(x) for x in xs]
        torch.cuda.synchronize()
        for _ in range(reps):
            dt.dt_allreduce(xs, ys)
            torch.cuda.synchronize()
        print(json.dumps({"probe_sweep": nbytes, "reps": reps, "alg_bytes_per_call": 2 * p * nbytes}), flush=True)
        del xs, ys
        torch.cuda.empty_cache()
    a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"probe": "done", "reps": reps, "copy_bytes_each_way": a.numel() * 4}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the one-timing-each pass over the other workloads (C1, C3, C4, C5)")
    ap.add_argument("--cpu-reps", type=int, default=25)
    ap.add_argument("--sweep", action="store_true", help="also run the P=16 size sweep and barrier latency")
    ap.add_argument("--probe", action="store_true", help="only run the kernels for a hardware-counter pass")
    ap.add_argument("--probe-rows", action="store_true",
                    help="only run the other rows' workloads once each (x3) for a hardware-counter pass")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="only run the P=16 sweep's HBM-resident AllReduces (x3) for a hardware-counter pass")
    ap.add_argument("--hsdp", action="store_true", help="also time the 32-layer gradient pipeline (103.6 GB)")
    ap.add_argument("--overlap", action="store_true", help="also run the GEMM / AllReduce overlap experiment")
    ap.add_argument("--coalescing", action="store_true", help="also compare the ways to reduce many small tensors")
    ap.add_argument("--all", action="store_true",
                    help="also time every other workload: small AllReduce, uneven AllGather, AllToAll, the size "
                         "sweep, the barrier and the gradient pipeline")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the same-device backend: all P logical ranks live on ONE GPU, so it runs "
              "on exactly one GPU (--gpus 1); multi-GPU runs are not part of this library.", file=sys.stderr)
        sys.exit(2)

    import torch
    import collective_communication_primitives_amd as dt
    import synth

    torch.cuda.set_device(0)
    if args.probe:
        probe(dt, torch)
        return
    if args.probe_rows:
        probe_rows(dt, torch)
        return
    if args.probe_sweep:
        probe_sweep(dt, torch)
        return
    stream = torch.cuda.current_stream()
    xs = synth.normal_ranks(P, SHAPE, seed=0, device="cuda", dtype=torch.bfloat16)
    n = SHAPE[0] * SHAPE[1]
    shards = [torch.empty(n // P, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    full = [torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    s_bytes = n * 2

    def rs():
        dt.dt_reduce_scatter(xs, shards)

    def ag():
        dt.dt_all_gather(shards, full)

    for _ in range(args.warmup):
        rs()
        ag()
    torch.cuda.synchronize()

    # timed region: K steps as a caller runs them, one event pair around all of
    # them on the stream the library launches on
    step_a, step_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_host0 = time.perf_counter()
    step_a.record(stream)
    for _ in range(args.steps):
        rs()
        ag()
    step_b.record(stream)
    torch.cuda.synchronize()
    t_host = time.perf_counter() - t_host0
    ms_total = step_a.elapsed_time(step_b)
    ms_per_step = ms_total / args.steps
    # the same K steps again, each launch bracketed by its own events: the
    # per-kernel durations of the roofline (the events add a few us per launch,
    # so these durations err long and the roofline fraction errs low)
    ev_rs, ev_ag = [], []
    sw_a, sw_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    sw_a.record(stream)
    for _ in range(args.steps):
        ev_rs += time_launches(rs, 1, stream)
        ev_ag += time_launches(ag, 1, stream)
    sw_b.record(stream)
    torch.cuda.synchronize()
    ms_per_step_events = sw_a.elapsed_time(sw_b) / args.steps
    rs_us = [a.elapsed_time(b) * 1e3 for a, b in ev_rs]
    ag_us = [a.elapsed_time(b) * 1e3 for a, b in ev_ag]

    algbw = s_bytes / (ms_per_step * 1e-3) / 1e9
    busbw = algbw * 2 * (P - 1) / P

    rs_bytes = (P + 1) * s_bytes          # read P inputs, write one shard per rank
    ag_bytes = (1 + P) * s_bytes          # read P shards, write P full outputs
    kernels = {
        "reduce_scatter": kernel_stats(rs_us, rs_bytes, s_bytes, (P - 1) / P),
        "all_gather": kernel_stats(ag_us, ag_bytes, s_bytes, (P - 1) / P),
    }
    dom_name = max(kernels, key=lambda k: kernels[k]["mean_us"])
    dom = kernels[dom_name]
    achieved = dom["alg_bytes"] / (dom["mean_us"] * 1e-6) / 1e9
    traffic = measured_traffic({"reduce_scatter": "reduce_scatter_bf16_p8", "all_gather": "all_gather_bf16_p8"}[dom_name])
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": dom_name,
                "alg_bytes_per_launch": dom["alg_bytes"]}

    # dt_allreduce on the same inputs, for reference; at 128 MiB per rank and P=8 it runs as a
    # ReduceScatter into each output's own chunk plus an in-place AllGather (two launches per call)
    ar_out = [torch.empty(SHAPE, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    for _ in range(args.warmup):
        dt.dt_allreduce(xs, ar_out)
    ev_ar = time_launches(lambda: dt.dt_allreduce(xs, ar_out), args.steps, stream)
    torch.cuda.synchronize()
    kernels["allreduce"] = kernel_stats([a.elapsed_time(b) * 1e3 for a, b in ev_ar], 2 * P * s_bytes,
                                        s_bytes, 2 * (P - 1) / P)
    del ar_out

    extra = {"kernels": kernels, "host_seconds_timed": round(t_host, 4), "kernel_source_hash": kernel_source_hash(),
             "ms_per_step_with_launch_events": round(ms_per_step_events, 4)}
    extra["int32_max"] = int32_max_step(dt, torch, args.steps, args.warmup, stream)
    extra["copy_ceiling"] = copy_ceiling(torch, stream)
    torch.cuda.empty_cache()
    if not args.no_configs:
        extra["configs"] = configs(dt, torch, steps=args.steps, warmup=2)
    if args.all:
        args.sweep = args.hsdp = args.overlap = args.coalescing = True
        extra["rows"] = other_rows(dt, torch, steps=args.steps, warmup=args.warmup)
    if args.sweep:
        rows, fit = sweep(dt, torch, steps=max(5, args.steps // 2), warmup=2)
        extra["sweep_p16_fp32"] = rows
        extra["alpha_beta_fit"] = fit
        extra["barrier"] = barrier_latency(dt, torch)
    if args.hsdp:
        extra["hsdp"] = hsdp(dt, torch)
    if args.overlap:
        extra["overlap"] = overlap(dt, torch)
    if args.coalescing:
        extra["coalescing"] = coalescing(dt, torch)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(xs, args.cpu_reps)

    line = {
        "metric": METRIC, "value": round(busbw, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "reduce_scatter_then_all_gather_bf16", "ranks": P, "shape_per_rank": list(SHAPE),
                   "op": "sum", "accumulate": "fp32", "seed": 0, "distribution": "N(0,1)",
                   "bytes_per_rank": s_bytes},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
