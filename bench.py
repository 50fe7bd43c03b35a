"""Benchmark of the TQ4_1S decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A *step* is one batch-1 decode pass over a Llama-3-8B-shaped model stored in
TQ4_1S: for each of the 32 layers and each activation group (q|k|v, o,
gate|up, down) the fused GEMV (tq_gemv, rotation fused) streams that group's
packed weights from HBM.  ``value`` is the whole step's algorithmic bytes
(0.625 B per weight + activations + outputs) divided by the step time, with
every input already resident in HBM.

The same run also measures, outside the timed step: the read envelope (a
plain streaming-read kernel over each group's bytes), the quantizer over the
whole model, the small-batch GEMM at M in {1, 4, 8, 16, 32, 64},
dequantization, the load-time int8 transcode and its decode step, NVFP4 /
MXFP6 quantize + decode on all 64 27B-shaped layers, the turbo4 KV-cache
decode attention, and the 80-layer Llama-3-70B quantize plus its FFN-trio
GEMV.  Every multi-launch row is captured in a HIP graph and replayed.
``roofline`` reports the dominant GEMV instantiation (HIP events on the
launch stream, and the committed rocprofv3 kernel statistics);
``cpu_baseline`` times the CPU oracle on a bounded sample on the host's
cores, before the GPU is initialised.  Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
WEIGHT_BYTES_PER_ELEM = 0.625      # 16 B nibbles + 4 B fp16 scales per 32 weights


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prerotate", action="store_true",
                    help="rotate each activation with tq_rotate before the GEMV instead of inside it")
    ap.add_argument("--no-graph", action="store_true", help="launch the step eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the CPU oracle sample")
    ap.add_argument("--layers27b", type=int, default=64, help="27B-shaped block-float layers (64 = the model)")
    return ap.parse_args()


def gemv_bytes(n, k, x_elem_bytes=2):
    """Algorithmic bytes of one GEMV: packed weights + activation + float32 output."""
    return WEIGHT_BYTES_PER_ELEM * n * k + x_elem_bytes * k + 4 * n


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# CPU oracle baseline.  Runs before anything touches the GPU; the all-cores
# figure uses a pool of fresh interpreters (spawn) over row chunks, each
# worker with one BLAS thread.
# ----------------------------------------------------------------------------

def _cpu_task(task):
    """One oracle call on a row chunk (pool worker): returns (seconds, result)."""
    from threadpoolctl import threadpool_limits

    from oracle import tq4_1s as otq
    kind = task[0]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if kind == "quant":
            res = otq.quantize_o32(task[1])
        else:
            otq.gemv_rows_o64(task[1], task[2], task[3])
            res = None
        return time.perf_counter() - t0, res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds):
    """The CPU oracle (float32 canonical quantizer, float64 GEMV) on a bounded sample of the workloads."""
    import multiprocessing as mp

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle import tq4_1s as otq

    cores = len(os.sched_getaffinity(0))
    procs = max(1, min(cores, 16))
    # Sample: the first R rows of one Llama-3-8B layer's four decode groups (float32 copies of the bf16
    # weights), plus the tiny round-trip workload whole.
    rows = 1024 if seconds >= 10 else 256
    members = {"qkv": ["q", "k", "v"], "o": ["o"], "gate_up": ["gate", "up"], "down": ["down"]}
    mats = {}
    for gname, names in members.items():
        mats[gname] = torch.cat([wl.llama8b_weight(t, 0, "cpu") for t in names], dim=0)[:rows].float().numpy()
    xs = {g: np.random.default_rng(i).standard_normal(m.shape[1]).astype(np.float32) for i, (g, m) in enumerate(mats.items())}
    chunk = 64
    qtasks = [("quant", m[r:r + chunk]) for m in mats.values() for r in range(0, rows, chunk)]
    q_weights = sum(m.size for m in mats.values())

    # single thread: quantize every chunk, then the GEMV of every chunk (repeated to the time budget)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        packed = [otq.quantize_o32(t[1]) for t in qtasks]
        q1 = time.perf_counter() - t0
    gtasks = []
    i = 0
    for gname, m in mats.items():
        for r in range(0, rows, chunk):
            p, s = packed[i]
            gtasks.append(("gemv", p, s, xs[gname]))
            i += 1
    g_bytes = sum(gemv_bytes(t[1].shape[0], t[1].shape[1] * 2, 4) for t in gtasks)
    reps = 1
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for t in gtasks:
            otq.gemv_rows_o64(t[1], t[2], t[3])
        g1 = time.perf_counter() - t0
    reps = max(1, int(min(seconds / 3, 8.0) / max(g1, 1e-3)))
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for _ in range(reps):
            for t in gtasks:
                otq.gemv_rows_o64(t[1], t[2], t[3])
        g1 = (time.perf_counter() - t0) / reps

    # all cores: the same chunks over a pool of fresh interpreters
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs) as pool:
        pool.map(_cpu_task, [("gemv",) + gtasks[0][1:]] * procs)          # interpreters and imports warm
        t0 = time.perf_counter()
        pool.map(_cpu_task, qtasks)
        qn = time.perf_counter() - t0
        t0 = time.perf_counter()
        for _ in range(reps):
            pool.map(_cpu_task, gtasks)
        gn = (time.perf_counter() - t0) / reps

    # the tiny round trip whole (single thread)
    W, x = wl.tiny_tq("cpu")
    with threadpool_limits(1):
        t0 = time.perf_counter()
        p, s = otq.quantize_o32(W.numpy())
        otq.gemv_rows_o64(p, s, x.numpy())
        tiny = time.perf_counter() - t0

    q_bytes = q_weights * (4 + WEIGHT_BYTES_PER_ELEM)                    # float32 in + packed out
    step_bytes = sum(32 * gemv_bytes(n, k) for n, k in wl.LLAMA8B_GROUPS.values())
    w70 = wl.LLAMA70B_LAYERS * sum(n * k for n, k in wl.LLAMA70B.values())
    return {
        "value": round(g_bytes / gn / 1e9, 4), "unit": "GB/s", "cores": procs, "kind": "oracle",
        "sample": (f"float64 oracle GEMV over the first {rows} rows of one Llama-3-8B layer's q|k|v, o, gate|up "
                   f"and down ({q_weights / 1e6:.1f} M weights, {len(gtasks)} chunks of {chunk} rows, a pool of "
                   f"{procs} processes with one BLAS thread each, {reps} passes)"),
        "host_cpus": cores, "cpu_model": _cpu_model(),
        "gemv_single_thread_GB_s": round(g_bytes / g1 / 1e9, 4),
        "gemv_all_cores_GB_s": round(g_bytes / gn / 1e9, 4),
        "quantize_single_thread_GB_s": round(q_bytes / q1 / 1e9, 4),
        "quantize_all_cores_GB_s": round(q_bytes / qn / 1e9, 4),
        "quantize_bytes": "4 B float32 in + 0.625 B out per weight (the oracle quantizes float32)",
        "tiny_256x512_round_trip_ms": round(tiny * 1e3, 2),
        "extrapolated": {
            "llama8b_step_s_all_cores": round(step_bytes / (g_bytes / gn), 2),
            "llama70b_quantize_h_all_cores": round(w70 * (4 + WEIGHT_BYTES_PER_ELEM) / (q_bytes / qn) / 3600, 2),
            "note": "per byte from the sample above; not measured whole",
        },
    }


# ----------------------------------------------------------------------------
# GPU helpers
# ----------------------------------------------------------------------------

def _graph(torch, fn):
    """Capture fn's launches (on torch's current stream) into a HIP graph after one eager warm-up."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _time(torch, stream, fn, reps):
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _time_graph(torch, stream, fn, reps, no_graph=False):
    """ms per call of fn, replayed from a HIP graph (or eagerly)."""
    if no_graph:
        return _time(torch, stream, fn, reps)
    g = _graph(torch, fn)
    ms = _time(torch, stream, g.replay, reps)
    del g
    return ms


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on exactly one GPU; "
                                   "multi-GPU sharding is described in the design notes but not built"}))
        sys.exit(2)

    cpu = None
    if not args.no_cpu_baseline:
        t = time.time()
        cpu = cpu_baseline(args.cpu_seconds)
        log(f"cpu baseline {time.time() - t:.1f}s")

    import torch
    import dequant_gemv_tq_amd as tqa
    import workloads as wl
    from dequant_gemv_tq_amd import profiling as tq_profiling

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    t_start = time.time()

    # ------------------------------------------------------------------ setup
    groups = wl.LLAMA8B_GROUPS                       # name -> (N, K)
    members = {"qkv": ["q", "k", "v"], "o": ["o"], "gate_up": ["gate", "up"], "down": ["down"]}
    L = wl.LLAMA8B_LAYERS
    model = []                                        # per layer: name -> (packed, scales)
    xs = []                                           # per layer: name -> bf16 activation
    # The bf16 model (14 GB) is drawn first; the quantizer then runs over all
    # 128 tensors back to back between two events on the launch stream.
    src = []
    for layer in range(L):
        variant = wl.layer_variant(layer)
        src.append({gname: torch.cat([wl.llama8b_weight(t, layer, dev, variant) for t in members[gname]], dim=0)
                    for gname in groups})
        g = wl.generator(wl.seed_of(2, layer, 50), dev)
        xs.append({gname: wl.activation(1, k, g, dev, torch.bfloat16)[0].contiguous()
                   for gname, (n, k) in groups.items()})
    for layer in range(L):
        model.append({gname: (torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                              torch.empty((n, k // 16), dtype=torch.int16, device=dev))
                      for gname, (n, k) in groups.items()})
    # One untimed call of each quantizer variant first, so that loading the
    # kernels' code objects stays out of the timed region.
    tqa.quantize(src[0]["o"], out=model[0]["o"])
    tqa.quantize(src[0]["o"], out=model[0]["o"], rsf=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for layer in range(L):
        for gname in groups:
            tqa.quantize(src[layer][gname], out=model[layer][gname])
    e1.record(stream)
    e1.synchronize()
    q_ms = e0.elapsed_time(e1)
    q_bytes = L * sum((2.0 + WEIGHT_BYTES_PER_ELEM) * n * k for n, k in groups.values())
    # RSF-lite scale search over the same tensors (offline quantizer option), and its error reduction.
    tmp = {gname: (torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                   torch.empty((n, k // 16), dtype=torch.int16, device=dev)) for gname, (n, k) in groups.items()}
    e0.record(stream)
    for layer in range(L):
        for gname in groups:
            tqa.quantize(src[layer][gname], out=tmp[gname], rsf=True)
    e1.record(stream)
    e1.synchronize()
    rsf_ms = e0.elapsed_time(e1)
    Wt = src[0]["gate_up"]
    Wf = Wt.float()
    err_plain = (tqa.dequantize(*model[0]["gate_up"]) - Wf).pow(2).sum().item()
    err_rsf = (tqa.dequantize(*tqa.quantize(Wt, rsf=True)) - Wf).pow(2).sum().item()
    rsf_row = {"GB_s": round(q_bytes / (rsf_ms * 1e-3) / 1e9, 1), "ms_total": round(rsf_ms, 3),
               "sq_error_vs_plain": round(err_rsf / err_plain, 4),
               "note": "nine scale multiples per half block; sq_error on layer 0 gate|up"}
    del src, tmp, Wf, Wt
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    xr_buf = {gname: torch.empty(k, dtype=torch.float32, device=dev) for gname, (n, k) in groups.items()}
    y_buf = {gname: torch.empty(n, dtype=torch.float32, device=dev) for gname, (n, k) in groups.items()}
    log(f"8B model ready {time.time() - t_start:.1f}s")

    step_bytes = 0.0
    for gname, (n, k) in groups.items():
        # fused: the GEMV reads the bf16 activation; prerotated: tq_rotate reads
        # 2K and writes 4K bytes, then the GEMV reads the 4K-byte x'
        step_bytes += L * (gemv_bytes(n, k, 2) if not args.prerotate else gemv_bytes(n, k, 4) + 6 * k)

    def launch_group(layer, gname):
        packed, scales = model[layer][gname]
        x = xs[layer][gname]
        if not args.prerotate:
            tqa.gemv(packed, scales, x, out=y_buf[gname])
        else:
            tqa.gemv(packed, scales, tqa.rotate(x, out=xr_buf[gname]), rotated=True, out=y_buf[gname])

    def step():
        for layer in range(L):
            for gname in groups:
                launch_group(layer, gname)

    # --------------------------------------------------------------- timed
    # The step's launches are captured once into a HIP graph (torch.cuda.graph
    # records on its capture stream, which is the current stream the library
    # launches on) and replayed; --no-graph launches them eagerly.  Each step
    # is bracketed by its own pair of events (no synchronisation between
    # steps) for the percentiles.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run_step = step
    if not args.no_graph:
        graph = _graph(torch, step)
        run_step = graph.replay
        for _ in range(max(1, args.warmup)):
            run_step()
        torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        run_step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms_per_step = evs[0].elapsed_time(evs[-1]) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    def pct(q):
        return per_step[min(len(per_step) - 1, int(round(q * (len(per_step) - 1))))]

    # ------------------------------------------------- per-launch GEMV timing
    # Each group's 32 launches (one per layer) are captured in a graph of
    # their own and replayed between two events on the launch stream: the
    # average launch duration of each GEMV shape (the gap to the next launch
    # included).  The read envelope is the same for a plain streaming-read
    # kernel over 32 distinct buffers of the group's packed bytes.
    xb = 2 if not args.prerotate else 4
    per_group, group_ms = {}, {}
    sink = torch.empty(tqa.STREAM_READ_SINK_WORDS, dtype=torch.int32, device=dev)
    for gname, (n, k) in groups.items():
        ms = _time_graph(torch, stream, lambda gname=gname: [launch_group(l_, gname) for l_ in range(L)], 5,
                         args.no_graph) / L
        nbytes = n * k // 2 + n * k // 8
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(L)]
        for b_ in bufs:
            b_.fill_(1)
        rms = _time_graph(torch, stream, lambda bufs=bufs: [tqa.stream_read(b_, sink=sink) for b_ in bufs], 5,
                          args.no_graph) / L
        del bufs
        group_ms[gname] = ms
        per_group[gname] = {"N": n, "K": k, "us": round(ms * 1e3, 2),
                            "GB_s": round(gemv_bytes(n, k, xb) / (ms * 1e-3) / 1e9, 1),
                            "read_envelope_us": round(rms * 1e3, 2),
                            "read_envelope_GB_s": round(nbytes / (rms * 1e-3) / 1e9, 1),
                            "gemv_over_read": round(ms / rms, 3)}
    torch.cuda.empty_cache()
    # Roofline of the dominant kernel: the instantiation that serves q|k|v, o
    # and gate|up (K = 4096, one row per wavefront; 96 of the 128 launches of
    # a step and 73% of its bytes).  down (K = 14336, activation rotated per
    # lane) is another instantiation.
    dom = list(tq_profiling.DOMINANT)
    dom_bytes = sum(gemv_bytes(groups[g][0], groups[g][1], xb) for g in dom)
    dom_ms = sum(group_ms[g] for g in dom)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    layer_kernel_ms = sum(group_ms.values())   # the four group launches of one layer
    # HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary,
    # and the kernel's average duration from the committed rocprofv3 kernel
    # statistics -- each None when taken from other kernel sources.
    rec = tq_profiling.read_record(os.path.join(ROOT, "profiles", "gemv_traffic_llama8b.md"))
    traffic = rec["traffic_bytes_per_launch"] if (rec and not args.prerotate) else None
    srec = tq_profiling.read_stats_record(os.path.join(ROOT, "profiles", "kernels_bench_llama8b.md"))
    rp_us = srec["kernels"].get(tq_profiling.DOMINANT_KERNEL) if (srec and not args.prerotate) else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": f"{tq_profiling.DOMINANT_KERNEL} (fused TQ4_1S GEMV, bf16 x, K = 4096)",
                "groups": dom, "launches_per_step": len(dom) * L,
                "bytes_per_launch_avg": round(dom_bytes / len(dom)),
                "avg_launch_us": round(dom_ms / len(dom) * 1e3, 2),
                "timing": "HIP events around graphs of each group's 32 launches (gap to the next launch included)",
                "rocprof_avg_us": rp_us,
                "rocprof_achieved": (round(dom_bytes / len(dom) / (rp_us * 1e-6) / 1e9, 1) if rp_us else None),
                "rocprof_frac": (round(dom_bytes / len(dom) / (rp_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                                 if rp_us else None)}
    log(f"8B step timed {time.time() - t_start:.1f}s")

    out = {
        "metric": "fused TQ4_1S GEMV achieved HBM GB/s (% of peak) at batch 1; quantize GB/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped 32-layer batch-1 decode, TQ4_1S weights, fused GEMV stream",
                   "layers": L, "groups": {g: list(v) for g, v in groups.items()},
                   "weights": "bf16 N(0,1/K) even layers, Student-t(4) odd layers, quantized on device",
                   "activation": "bf16 [K] N(0,1), one per group and layer",
                   "rotation": "fused in GEMV" if (not args.prerotate) else "tq_rotate + tq_gemv",
                   "launch": "eager" if args.no_graph else "HIP graph replay",
                   "step_bytes": int(step_bytes)},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "step_ms_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4), round(pct(0.9), 4)],
        "tokens_equiv_layers_per_s": round(1e3 / layer_kernel_ms, 1),
        "tokens_per_s_32_layers": round(1e3 / ms_per_step, 2),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "per_group": per_group,
        "read_envelope_step_ms": round(L * sum(per_group[g]["read_envelope_us"] for g in groups) / 1e3, 4),
        "quantize": {"GB_s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "ms_total": round(q_ms, 3),
                     "weights": int(q_bytes / (2.0 + WEIGHT_BYTES_PER_ELEM)),
                     "bytes": "2 B bf16 in + 0.625 B out per weight",
                     "timing": "128 tensors of the bf16 model quantized back to back between two events",
                     "rsf": rsf_row},
    }

    # ----------------------------------------------------- secondary rows
    out["gemm"] = bench_gemm(torch, tqa, wl, model, groups, dev, stream, args.no_graph)
    out["dequantize"] = bench_dequant(torch, tqa, model, groups, dev, stream)
    out["q8_transcode"] = bench_q8(torch, tqa, model, xs, groups, dev, stream, ms_per_step, args.no_graph)
    log(f"8B secondary rows {time.time() - t_start:.1f}s")
    del model, xs
    torch.cuda.empty_cache()
    out["blockfp"] = bench_blockfp(torch, tqa, wl, dev, stream, args.layers27b, args.no_graph)
    log(f"27B block-float rows {time.time() - t_start:.1f}s")
    out["kv_attention"] = bench_kv(torch, tqa, wl, dev, stream, args.no_graph)
    log(f"kv rows {time.time() - t_start:.1f}s")
    out["llama70b"] = bench_70b(torch, tqa, wl, dev, stream, args.no_graph)
    log(f"70B rows {time.time() - t_start:.1f}s")
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def bench_gemm(torch, tqa, wl, model, groups, dev, stream, no_graph):
    """Small-batch GEMM over the 32-layer stream (bf16 pre-rotated activations), graph-replayed."""
    res = {}
    L = len(model)
    for m in (1, 4, 8, 16, 32, 64):
        xr = {}
        for gi, (gname, (n, k)) in enumerate(groups.items()):
            g = wl.generator(wl.seed_of(3, m, gi), dev)
            X = wl.activation(m, k, g, dev, torch.bfloat16)
            xr[gname] = tqa.rotate(X, dtype=torch.bfloat16)
        ys = {gname: torch.empty((m, n), dtype=torch.float32, device=dev) for gname, (n, k) in groups.items()}

        def run():
            for layer in range(L):
                for gname in groups:
                    p, s = model[layer][gname]
                    tqa.gemm(p, s, xr[gname], out=ys[gname])

        ms = _time_graph(torch, stream, run, 3, no_graph)
        byts = sum(L * (WEIGHT_BYTES_PER_ELEM * n * k + 2 * m * k + 4 * m * n) for n, k in groups.values())
        flops = sum(L * 2.0 * m * n * k for n, k in groups.values())
        res[f"M{m}"] = {"ms_32_layers": round(ms, 3), "GB_s": round(byts / (ms * 1e-3) / 1e9, 1),
                        "TFLOP_s": round(flops / (ms * 1e-3) / 1e12, 2),
                        "path": "VALU fp32" if m <= 2 else "MFMA bf16"}
    return res


def bench_dequant(torch, tqa, model, groups, dev, stream):
    n, k = groups["gate_up"]
    p, s = model[0]["gate_up"]
    out = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
    ms = _time(torch, stream, lambda: tqa.dequantize(p, s, dtype=torch.bfloat16, out=out), 5)
    byts = (WEIGHT_BYTES_PER_ELEM + 2.0) * n * k
    return {"shape": [n, k], "out": "bf16", "us": round(ms * 1e3, 1), "GB_s": round(byts / (ms * 1e-3) / 1e9, 1)}


def bench_q8(torch, tqa, model, xs, groups, dev, stream, tq4_ms, no_graph):
    """Load-time TQ4_1S -> int8 transcode of the 32-layer model, then the int8 decode step (same launches
    and activations as the TQ4_1S step: one q8 GEMV per group and layer, captured in a graph)."""
    L = len(model)
    # Outputs allocated first and one untimed call, so that the timed region
    # holds the 128 transcodes back to back and nothing else.
    q8 = [{gname: (torch.empty((n, k), dtype=torch.int8, device=dev),
                   torch.empty((n, k // 32), dtype=torch.int16, device=dev))
           for gname, (n, k) in groups.items()} for _ in range(L)]
    tqa.transcode_q8(*model[0]["o"], out=q8[0]["o"])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for layer in range(L):
        for gname in groups:
            tqa.transcode_q8(*model[layer][gname], out=q8[layer][gname])
    b.record(stream)
    b.synchronize()
    q_ms = a.elapsed_time(b)
    q_weights = L * sum(n * k for n, k in groups.values())
    ys = {gname: torch.empty(n, dtype=torch.float32, device=dev) for gname, (n, k) in groups.items()}

    def step():
        for layer in range(L):
            for gname in groups:
                c, qs = q8[layer][gname]
                tqa.q8_gemv(c, qs, xs[layer][gname], out=ys[gname])

    ms = _time_graph(torch, stream, step, 10, no_graph)
    byts = sum(L * (1.0625 * n * k + 2 * k + 4 * n) for n, k in groups.values())
    res = {"transcode_GB_s": round((WEIGHT_BYTES_PER_ELEM + 1.0625) * q_weights / (q_ms * 1e-3) / 1e9, 1),
           "transcode_ms_total": round(q_ms, 3), "bytes_per_weight": 1.0625,
           "gemv_step_ms": round(ms, 4), "gemv_GB_s": round(byts / (ms * 1e-3) / 1e9, 1),
           "gemv_step_time_vs_tq4": round(ms / tq4_ms, 3),
           "note": "int8 codes + fp16 block scales; activation quantized to int8 per block inside the GEMV"}
    del q8
    torch.cuda.empty_cache()
    return res


BF_BYTES = {"nvfp4": 0.5625, "mxfp6": 0.78125}


def bench_blockfp(torch, tqa, wl, dev, stream, layers, no_graph):
    """27B-shaped layers (all 64 by default): per-tensor NVFP4 or MXFP6 (seeded, ~10% MXFP6); quantize, and
    the fused decode at M = 1 (VALU GEMV), 8, 16 and 64 (bf16 MFMA), graph-replayed, over the loader's
    layout (same-format q|k|v and gate|up members concatenated) and over one launch per tensor."""
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    fmt_count = {"nvfp4": 0, "mxfp6": 0}
    src = []
    for layer in range(layers):
        for t in names:
            fmt = wl.qwen27b_format(layer, t)
            fmt_count[fmt] += 1
            src.append((fmt, wl.qwen27b_weight(t, layer, dev)))
    # Outputs and workspace allocated first; an untimed pass loads the kernels.
    outs = []
    for fmt, W in src:
        n, k = W.shape
        if fmt == "nvfp4":
            outs.append((torch.empty((n, k // 2), dtype=torch.uint8, device=dev),
                         torch.empty((n, k // 16), dtype=torch.uint8, device=dev),
                         torch.empty(1, dtype=torch.float32, device=dev)))
        else:
            outs.append((torch.empty((n, 3 * k // 4), dtype=torch.uint8, device=dev),
                         torch.empty((n, k // 32), dtype=torch.uint8, device=dev), None))
    ws = torch.empty(tqa.workspace_bytes("nvfp4_quantize", 1, 16), dtype=torch.uint8, device=dev)
    for fmt in fmt_count:
        i = next((i for i, (f, _) in enumerate(src) if f == fmt), None)
        if i is not None:
            tqa.blockfp_quantize(fmt, src[i][1], workspace=ws, out=outs[i])
            tqa.blockfp_quantize(fmt, src[i][1], rsf=True, workspace=ws, out=outs[i])
    torch.cuda.synchronize()
    q_bytes = sum((2.0 * (2 if f == "nvfp4" else 1) + BF_BYTES[f]) * W.numel() for f, W in src)

    def quant(rsf):
        for (fmt, W), o in zip(src, outs):
            tqa.blockfp_quantize(fmt, W, rsf=rsf, workspace=ws, out=o)

    rsf_ms = _time(torch, stream, lambda: quant(True), 1)
    q_ms = _time(torch, stream, lambda: quant(False), 1)        # last, so the outputs hold the plain codes
    store = [(fmt, c, bs, ts, W.shape[0], W.shape[1]) for (fmt, W), (c, bs, ts) in zip(src, outs)]
    # The fused layout: per layer, the members of q|k|v and of gate|up that share a format are stored as
    # one row-concatenated tensor (one NVFP4 tensor scale for the concatenation), as one decode launch
    # reads them; o and down stay alone.  Quantized here untimed, one layer at a time.
    fused = []
    fgroups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    for layer in range(layers):
        mine = dict(zip(names, src[layer * len(names):(layer + 1) * len(names)]))
        for grp in fgroups:
            for fmt in ("nvfp4", "mxfp6"):
                parts = [mine[t][1] for t in grp if mine[t][0] == fmt]
                if not parts:
                    continue
                Wc = torch.cat(parts, dim=0) if len(parts) > 1 else parts[0]
                c, bs, ts = tqa.blockfp_quantize(fmt, Wc, workspace=ws)
                fused.append((fmt, c, bs, ts, Wc.shape[0], Wc.shape[1]))
                del Wc
    del src
    torch.cuda.empty_cache()
    res = {"layers": layers, "tensors": fmt_count, "quantize_GB_s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
           "quantize_ms": round(q_ms, 2), "quantize_rsf_GB_s": round(q_bytes / (rsf_ms * 1e-3) / 1e9, 1),
           "quantize_bytes": "NVFP4 reads the bf16 weights twice (amax, encode); MXFP6 once",
           "quantize_launches": "NVFP4: amax + encode; MXFP6: encode"}
    # gemv_M{m}: the layout a loader produces (same-format members of q|k|v and of gate|up
    # row-concatenated, one launch each); gemv_M{m}_per_tensor: one launch per tensor, for contrast.
    res["layout"] = "gemv_M*: same-format members of q|k|v and of gate|up row-concatenated; o and down alone"
    for m in (1, 8, 16, 64):
        xsv = {}
        for (fmt, codes, bs, ts, n, k) in store:
            if k not in xsv:
                g = wl.generator(wl.seed_of(4, m, k), dev)
                xsv[k] = wl.activation(m, k, g, dev, torch.bfloat16)
        for key, tensors in ((f"gemv_M{m}", fused), (f"gemv_M{m}_per_tensor", store)):
            ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for (_, _, _, _, n, _) in tensors]

            def run(tensors=tensors, ys=ys):
                for i, (fmt, codes, bs, ts, n, k) in enumerate(tensors):
                    tqa.blockfp_gemm(fmt, codes, bs, ts, xsv[k], out=ys[i])

            ms = _time_graph(torch, stream, run, 3, no_graph)
            byts = sum((BF_BYTES[f] * n * k + 2 * m * k + 4 * m * n) for (f, _, _, _, n, k) in tensors)
            res[key] = {"ms": round(ms, 3), "GB_s": round(byts / (ms * 1e-3) / 1e9, 1), "launches": len(tensors)}
            del ys
    del store, fused
    torch.cuda.empty_cache()
    return res


KV_BYTES = 128 + 8 + 64 + 2      # per cached token and cache head: q8_0 key codes + scales, turbo4 nibbles + norm


def bench_kv(torch, tqa, wl, dev, stream, no_graph, layers=32, batch=16, ctx=4096):
    """turbo4 V / q8_0 K cache of the Llama-3-8B attention layout (32 query heads, 8 cache heads, head dim
    128): bulk encode of every layer's cache, then one decode-attention step over all layers (split kernel +
    combine per layer, captured in a graph), batch 16 x 4096 cached tokens."""
    Hq, Hkv, D = 32, 8, 128
    caches, enc_ms = [], 0.0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for layer in range(layers):
        g = wl.generator(wl.seed_of(6, layer, 0), dev)
        K = torch.randn((batch, Hkv, ctx, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        V = torch.randn((batch, Hkv, ctx, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        kc = torch.empty(K.shape, dtype=torch.int8, device=dev)
        ks = torch.empty(K.shape[:-1] + (D // 32,), dtype=torch.int16, device=dev)
        vp = torch.empty(V.shape[:-1] + (D // 2,), dtype=torch.uint8, device=dev)
        vn = torch.empty(V.shape[:-1], dtype=torch.int16, device=dev)
        if layer == 0:                       # untimed: kernels loaded before the first timed encode
            tqa.kv_quantize_k(K, out=(kc, ks))
            tqa.kv_quantize_v(V, out=(vp, vn))
        torch.cuda.synchronize()
        a.record(stream)
        tqa.kv_quantize_k(K, out=(kc, ks))
        tqa.kv_quantize_v(V, out=(vp, vn))
        b.record(stream)
        b.synchronize()
        enc_ms += a.elapsed_time(b)
        caches.append((kc, ks, vp, vn))
        del K, V
    torch.cuda.empty_cache()
    g = wl.generator(wl.seed_of(6, 99, 1), dev)
    qs = [torch.randn((batch, Hq, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
          for _ in range(layers)]
    lengths = torch.full((batch,), ctx, dtype=torch.int32, device=dev)
    outs = [torch.empty((batch, Hq, D), dtype=torch.float32, device=dev) for _ in range(layers)]
    ws = torch.empty(tqa.attn_workspace_bytes(batch, Hq, ctx), dtype=torch.uint8, device=dev)
    sign = tqa.kv_sign_from_seed(0)

    def step():
        for layer in range(layers):
            kc, ks, vp, vn = caches[layer]
            tqa.attn_decode(qs[layer], lengths, kc, ks, vp, vn, sign=sign, out=outs[layer], workspace=ws)

    ms = _time_graph(torch, stream, step, 10, no_graph)
    kv_bytes = layers * batch * ctx * Hkv * KV_BYTES
    byts = kv_bytes + layers * batch * Hq * D * (2 + 4)
    elems = layers * batch * ctx * Hkv * D
    del caches
    torch.cuda.empty_cache()
    return {"layout": {"layers": layers, "batch": batch, "context": ctx, "q_heads": Hq, "kv_heads": Hkv,
                       "head_dim": D},
            "encode_GB_s": round(2 * elems * (2 + KV_BYTES / (2 * D)) / (enc_ms * 1e-3) / 1e9, 1),
            "decode_step_ms": round(ms, 3), "decode_GB_s": round(byts / (ms * 1e-3) / 1e9, 1),
            "cache_bytes_per_token_head": KV_BYTES, "bf16_cache_bytes_per_token_head": 2 * 2 * D,
            "note": "decode GB/s counts the quantized cache + q + o; the split kernel's partials are extra"}


def bench_70b(torch, tqa, wl, dev, stream, no_graph, gemv_layers=3):
    """Llama-3-70B shapes, per-layer std drift U(0.5, 2): all 80 layers quantized (each tensor drawn on the
    device untimed, quantized between two events, freed), then the batch-1 fused GEMV over the FFN trio
    (gate|up row-concatenated, one bf16 activation, and down) of several layers, graph-replayed."""
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    q_ms, weights = 0.0, 0
    keep = []
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    first = True
    for layer in range(wl.LLAMA70B_LAYERS):
        ffn = {}
        for t in names:
            W = wl.llama70b_weight(t, layer, dev)
            n, k = W.shape
            p = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
            s = torch.empty((n, k // 16), dtype=torch.int16, device=dev)
            if first:                           # untimed: kernel loaded before the first timed call
                tqa.quantize(W, out=(p, s))
                first = False
            torch.cuda.synchronize()
            a.record(stream)
            tqa.quantize(W, out=(p, s))
            b.record(stream)
            b.synchronize()
            q_ms += a.elapsed_time(b)
            weights += n * k
            if layer < gemv_layers and t in ("gate", "up", "down"):
                ffn[t] = (p, s)
            del W
        if ffn:
            gu = (torch.cat([ffn["gate"][0], ffn["up"][0]], dim=0), torch.cat([ffn["gate"][1], ffn["up"][1]], dim=0))
            keep.append({"gate_up": gu, "down": ffn["down"]})
        del ffn
    torch.cuda.empty_cache()
    res = {"layers": wl.LLAMA70B_LAYERS, "weights": weights, "quantize_ms": round(q_ms, 1),
           "quantize_GB_s": round((2.0 + WEIGHT_BYTES_PER_ELEM) * weights / (q_ms * 1e-3) / 1e9, 1),
           "quantize_timing": "sum over the 560 tensors of one event pair each (drawn on the device between)"}
    shapes = {"gate_up": (2 * wl.LLAMA70B["gate"][0], wl.LLAMA70B["gate"][1]), "down": wl.LLAMA70B["down"]}
    xs = [{g: wl.activation(1, k, wl.generator(wl.seed_of(5, li, 77 + gi), dev), dev, torch.bfloat16)[0].contiguous()
           for gi, (g, (n, k)) in enumerate(shapes.items())} for li in range(len(keep))]
    ys = {g: torch.empty(n, dtype=torch.float32, device=dev) for g, (n, k) in shapes.items()}
    per = {}
    for g, (n, k) in shapes.items():
        ms = _time_graph(torch, stream, lambda g=g: [tqa.gemv(*keep[i][g], xs[i][g], out=ys[g])
                                                     for i in range(len(keep))], 10, no_graph) / len(keep)
        per[g] = {"N": n, "K": k, "us": round(ms * 1e3, 2), "GB_s": round(gemv_bytes(n, k) / (ms * 1e-3) / 1e9, 1)}
    # Kernel execution time of gate|up from the committed rocprofv3 kernel statistics (None when they were
    # taken from other sources): in this benchmark the K = 8192 instantiation serves this matrix alone.
    from dequant_gemv_tq_amd import profiling as tq_profiling
    srec = tq_profiling.read_stats_record(os.path.join(ROOT, "profiles", "kernels_bench_llama8b.md"))
    rp = srec["kernels"].get(tq_profiling.GATE_UP_70B_KERNEL) if srec else None
    n, k = shapes["gate_up"]
    per["gate_up"]["rocprof_kernel"] = tq_profiling.GATE_UP_70B_KERNEL
    per["gate_up"]["rocprof_us"] = rp
    per["gate_up"]["rocprof_frac"] = (round(gemv_bytes(n, k) / (rp * 1e-6) / 1e9 / PEAK_HBM_GBS, 4) if rp else None)
    trio_ms = _time_graph(torch, stream, lambda: [tqa.gemv(*keep[i][g], xs[i][g], out=ys[g]) for i in range(len(keep))
                                                  for g in shapes], 10, no_graph) / len(keep)
    trio_bytes = sum(gemv_bytes(n, k) for n, k in shapes.values())
    res["ffn_trio_gemv"] = {"packed_GB": round(sum(WEIGHT_BYTES_PER_ELEM * n * k for n, k in shapes.values()) / 1e9, 3),
                            "layers_streamed": len(keep), "us_per_layer": round(trio_ms * 1e3, 1),
                            "GB_s": round(trio_bytes / (trio_ms * 1e-3) / 1e9, 1),
                            "pct_of_peak": round(100 * trio_bytes / (trio_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
                            "per_launch": per, "activation": "bf16 [K], rotation fused"}
    del keep
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
