"""Benchmark of the TQ4_1S decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extended]

A *step* is one batch-1 decode pass over a Llama-3-8B-shaped model stored in
TQ4_1S: for each of the 32 layers and each activation group (q|k|v, o,
gate|up, down) the activation is rotated once (tq_rotate) and the fused GEMV
(tq_gemv) streams that group's packed weights from HBM.  ``value`` is the
whole step's algorithmic bytes (0.625 B per weight + activations + outputs)
divided by the step time, with every input already resident in HBM.

The same run also measures, outside the timed step: the quantizer over the
whole model, the small-batch GEMM at M in {1, 4, 16, 32, 64}, dequantization,
the load-time int8 transcode of the model and its int8 decode step,
and NVFP4 / MXFP6 quantize + GEMV on 27B-shaped layers (a few layers by
default, all 64 plus the 70B quantize with --extended).  ``roofline``
reports the fused GEMV kernel alone (per-launch HIP event pairs on the
launch stream); ``cpu_baseline`` times the CPU oracle on a bounded sample.
Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
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
    ap.add_argument("--extended", action="store_true", help="all 64 27B layers and the 80-layer 70B quantize")
    ap.add_argument("--prerotate", action="store_true",
                    help="rotate each activation with tq_rotate before the GEMV instead of inside it")
    ap.add_argument("--no-graph", action="store_true", help="launch the step eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def gemv_bytes(n, k, x_elem_bytes=4):
    """Algorithmic bytes of one GEMV: packed weights + activation + float32 output."""
    return WEIGHT_BYTES_PER_ELEM * n * k + x_elem_bytes * k + 4 * n


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": f"--gpus {args.gpus}: this benchmark runs on exactly one GPU; "
                                   "multi-GPU sharding is described in the design notes but not built"}))
        sys.exit(2)

    import torch
    import dequant_gemv_tq_amd as tqa
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

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
    del src, tmp, Wf
    torch.cuda.empty_cache()
    torch.cuda.synchronize()
    xr_buf = {gname: torch.empty(k, dtype=torch.float32, device=dev) for gname, (n, k) in groups.items()}
    y_buf = {gname: torch.empty(n, dtype=torch.float32, device=dev) for gname, (n, k) in groups.items()}

    step_bytes = 0.0
    for gname, (n, k) in groups.items():
        # fused: the GEMV reads the bf16 activation; prerotated: tq_rotate reads
        # 2K and writes 4K bytes, then the GEMV reads the 4K-byte x'
        step_bytes += L * (gemv_bytes(n, k, 2) if not args.prerotate else gemv_bytes(n, k, 4) + 6 * k)

    def step():
        for layer in range(L):
            for gname in groups:
                packed, scales = model[layer][gname]
                x = xs[layer][gname]
                if not args.prerotate:
                    tqa.gemv(packed, scales, x, out=y_buf[gname])
                else:
                    xr = tqa.rotate(x, out=xr_buf[gname])
                    tqa.gemv(packed, scales, xr, rotated=True, out=y_buf[gname])

    # --------------------------------------------------------------- timed
    # The step's launches are captured once into a HIP graph (torch.cuda.graph
    # records on its capture stream, which is the current stream the library
    # launches on) and replayed; --no-graph launches them eagerly.
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run_step = step
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run_step = graph.replay
        for _ in range(max(1, args.warmup)):
            run_step()
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ------------------------------------------------- per-launch GEMV timing
    # Each group's 32 launches (one per layer) are captured in a graph of
    # their own and replayed between two events on the launch stream: the
    # average launch duration of each GEMV shape.
    xb = 2 if not args.prerotate else 4
    per_group = {}
    group_ms = {}
    for gname, (n, k) in groups.items():
        def group_step(gname=gname):
            for layer in range(L):
                packed, scales = model[layer][gname]
                x = xs[layer][gname]
                if not args.prerotate:
                    tqa.gemv(packed, scales, x, out=y_buf[gname])
                else:
                    tqa.gemv(packed, scales, tqa.rotate(x, out=xr_buf[gname]), rotated=True, out=y_buf[gname])
        if args.no_graph:
            ms = _time(torch, stream, group_step, 5) / L
        else:
            gg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gg):
                group_step()
            ms = _time(torch, stream, gg.replay, 5) / L
            del gg
        group_ms[gname] = ms
        per_group[gname] = {"N": n, "K": k, "us": round(ms * 1e3, 2),
                            "GB_s": round(gemv_bytes(n, k, xb) / (ms * 1e-3) / 1e9, 1)}
    # Roofline of the dominant kernel: the instantiation that serves q|k|v and
    # gate|up (K = 4096, one row per wavefront; 64 of the 128 launches of a
    # step and 57% of its bytes).  o (one two-row tile per workgroup) and down
    # (K = 14336, activation staged in four passes) are other instantiations.
    from dequant_gemv_tq_amd import profiling as tq_profiling
    dom = list(tq_profiling.DOMINANT)
    dom_bytes = sum(gemv_bytes(groups[g][0], groups[g][1], xb) for g in dom)
    dom_ms = sum(group_ms[g] for g in dom)
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    layer_kernel_ms = sum(group_ms.values())   # the four group launches of one layer
    # HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary,
    # or None when it was taken from other kernel sources than these.
    rec = tq_profiling.read_record(os.path.join(ROOT, "profiles", "gemv_traffic_llama8b.md"))
    traffic = rec["traffic_bytes_per_launch"] if (rec and not args.prerotate) else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": f"{tq_profiling.DOMINANT_KERNEL} (fused TQ4_1S GEMV, bf16 x, K = 4096)",
                "groups": dom, "launches_per_step": len(dom) * L,
                "bytes_per_launch_avg": round(dom_bytes / len(dom)),
                "avg_launch_us": round(dom_ms / len(dom) * 1e3, 2)}

    out = {
        "metric": "fused TQ4_1S GEMV achieved HBM GB/s (% of peak) at batch 1; quantize GB/s",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Llama-3-8B-shaped 32-layer batch-1 decode, TQ4_1S weights, fused GEMV stream",
                   "layers": L, "groups": {g: list(v) for g, v in groups.items()},
                   "weights": "bf16 N(0,1/K) even layers, Student-t(4) odd layers, quantized on device",
                   "activation": "bf16 [K] N(0,1), rotated once per group",
                   "rotation": "fused in GEMV" if (not args.prerotate) else "tq_rotate + tq_gemv",
                   "launch": "eager" if args.no_graph else "HIP graph replay",
                   "step_bytes": int(step_bytes)},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "tokens_equiv_layers_per_s": round(1e3 / layer_kernel_ms, 1),
        "tokens_per_s_32_layers": round(1e3 / ms_per_step, 2),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "per_group": per_group,
        "quantize": {"GB_s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1), "ms_total": round(q_ms, 3),
                     "weights": int(q_bytes / (2.0 + WEIGHT_BYTES_PER_ELEM)),
                     "bytes": "2 B bf16 in + 0.625 B out per weight",
                     "timing": "128 tensors of the bf16 model quantized back to back between two events",
                     "rsf": rsf_row},
    }

    # ----------------------------------------------------- secondary rows
    out["gemm"] = bench_gemm(torch, tqa, wl, model, groups, dev, stream)
    out["dequantize"] = bench_dequant(torch, tqa, model, groups, dev, stream)
    out["q8_transcode"] = bench_q8(torch, tqa, model, xs, groups, dev, stream, ms_per_step, args.no_graph)
    out["blockfp"] = bench_blockfp(torch, tqa, wl, dev, stream, layers=64 if args.extended else 4)
    out["kv_attention"] = bench_kv(torch, tqa, wl, dev, stream, args.no_graph)
    if args.extended:
        del model, xs
        torch.cuda.empty_cache()
        out["llama70b"] = bench_70b(torch, tqa, wl, dev, stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(model, groups, args.cpu_seconds)
    print(json.dumps(out), flush=True)


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


def bench_gemm(torch, tqa, wl, model, groups, dev, stream):
    """Small-batch GEMM over the 32-layer stream (bf16 pre-rotated activations)."""
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

        ms = _time(torch, stream, run, 3)
        byts = sum(L * (WEIGHT_BYTES_PER_ELEM * n * k + 2 * m * k + 4 * m * n) for n, k in groups.values())
        flops = sum(L * 2.0 * m * n * k for n, k in groups.values())
        res[f"M{m}"] = {"ms_32_layers": round(ms, 3), "GB_s": round(byts / (ms * 1e-3) / 1e9, 1),
                        "TFLOP_s": round(flops / (ms * 1e-3) / 1e12, 2),
                        "path": "VALU fp32" if m <= 4 else "MFMA bf16"}
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

    if no_graph:
        ms = _time(torch, stream, step, 5)
    else:
        step()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        ms = _time(torch, stream, gr.replay, 10)
        del gr
    byts = sum(L * (1.0625 * n * k + 2 * k + 4 * n) for n, k in groups.values())
    res = {"transcode_GB_s": round((WEIGHT_BYTES_PER_ELEM + 1.0625) * q_weights / (q_ms * 1e-3) / 1e9, 1),
           "transcode_ms_total": round(q_ms, 3), "bytes_per_weight": 1.0625,
           "gemv_step_ms": round(ms, 4), "gemv_GB_s": round(byts / (ms * 1e-3) / 1e9, 1),
           "gemv_step_time_vs_tq4": round(ms / tq4_ms, 3),
           "note": "int8 codes + fp16 block scales; activation quantized to int8 per block inside the GEMV"}
    del q8
    torch.cuda.empty_cache()
    return res


def bench_blockfp(torch, tqa, wl, dev, stream, layers):
    """27B-shaped layers: per-tensor NVFP4 or MXFP6 (seeded, ~10% MXFP6); quantize, and the fused decode at
    M = 1 (VALU GEMV), 8, 16 and 64 (bf16 MFMA)."""
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    store = []
    q_bytes = 0.0
    fmt_count = {"nvfp4": 0, "mxfp6": 0}
    src = []
    for layer in range(layers):
        for t in names:
            fmt = wl.qwen27b_format(layer, t)
            fmt_count[fmt] += 1
            src.append((fmt, wl.qwen27b_weight(t, layer, dev)))
    # An untimed pass first: it loads the kernels and leaves the outputs'
    # blocks in torch's caching allocator, so the timed passes allocate nothing.
    warm = [tqa.blockfp_quantize(fmt, W) for fmt, W in src]
    for fmt in fmt_count:
        first = next((W for f, W in src if f == fmt), None)
        if first is not None:
            warm.append(tqa.blockfp_quantize(fmt, first, rsf=True))
    del warm
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)                                    # all tensors back to back between two events
    for fmt, W in src:
        n, k = W.shape
        codes, bs, ts = tqa.blockfp_quantize(fmt, W)
        reads = 2 if fmt == "nvfp4" else 1              # NVFP4 reads W twice (amax, encode)
        q_bytes += (2.0 * reads + (0.5625 if fmt == "nvfp4" else 0.78125)) * n * k
        store.append((fmt, codes, bs, ts, n, k))
    b.record(stream)
    b.synchronize()
    q_ms = a.elapsed_time(b)
    a.record(stream)                                    # the same tensors with the RSF-lite block-scale search
    for fmt, W in src:
        tqa.blockfp_quantize(fmt, W, rsf=True)
    b.record(stream)
    b.synchronize()
    rsf_ms = a.elapsed_time(b)
    del src
    torch.cuda.empty_cache()
    res = {"layers": layers, "tensors": fmt_count, "quantize_GB_s": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
           "quantize_rsf_GB_s": round(q_bytes / (rsf_ms * 1e-3) / 1e9, 1)}
    for m in (1, 8, 16, 64):
        xsv = {}
        for (fmt, codes, bs, ts, n, k) in store:
            if k not in xsv:
                g = wl.generator(wl.seed_of(4, m, k), dev)
                xsv[k] = wl.activation(m, k, g, dev, torch.bfloat16)
        ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for (_, _, _, _, n, _) in store]

        def run():
            for i, (fmt, codes, bs, ts, n, k) in enumerate(store):
                tqa.blockfp_gemm(fmt, codes, bs, ts, xsv[k], out=ys[i])

        ms = _time(torch, stream, run, 3)
        byts = sum(((0.5625 if f == "nvfp4" else 0.78125) * n * k + 2 * m * k + 4 * m * n)
                   for (f, _, _, _, n, k) in store)
        res[f"gemv_M{m}"] = {"ms": round(ms, 3), "GB_s": round(byts / (ms * 1e-3) / 1e9, 1)}
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

    run = step
    if not no_graph:
        step()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        run = gr.replay
    ms = _time(torch, stream, run, 10)
    kv_bytes = layers * batch * ctx * Hkv * KV_BYTES
    byts = kv_bytes + layers * batch * Hq * D * (2 + 4)
    elems = layers * batch * ctx * Hkv * D
    return {"layout": {"layers": layers, "batch": batch, "context": ctx, "q_heads": Hq, "kv_heads": Hkv,
                       "head_dim": D},
            "encode_GB_s": round(2 * elems * (2 + KV_BYTES / (2 * D)) / (enc_ms * 1e-3) / 1e9, 1),
            "decode_step_ms": round(ms, 3), "decode_GB_s": round(byts / (ms * 1e-3) / 1e9, 1),
            "cache_bytes_per_token_head": KV_BYTES, "bf16_cache_bytes_per_token_head": 2 * 2 * D,
            "note": "decode GB/s counts the quantized cache + q + o; the split kernel's partials are extra"}


def bench_70b(torch, tqa, wl, dev, stream):
    """Full 80-layer 70B-shaped quantize (generated one tensor at a time) and the FFN-trio GEMV."""
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    q_ms, weights = 0.0, 0
    keep = None
    for layer in range(wl.LLAMA70B_LAYERS):
        for t in names:
            W = wl.llama70b_weight(t, layer, dev)
            n, k = W.shape
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            p, s = tqa.quantize(W)
            b.record(stream)
            b.synchronize()
            q_ms += a.elapsed_time(b)
            weights += n * k
            if layer == 0 and t in ("gate", "up", "down"):
                keep = (keep or {})
                keep[t] = (p, s, n, k)
            del W, p, s
    res = {"weights": weights, "quantize_ms": round(q_ms, 1),
           "quantize_GB_s": round((2.0 + WEIGHT_BYTES_PER_ELEM) * weights / (q_ms * 1e-3) / 1e9, 1)}
    xr = {}
    for t, (p, s, n, k) in keep.items():
        g = wl.generator(wl.seed_of(5, 0, 77), dev)
        xr[t] = tqa.rotate(wl.activation(1, k, g, dev, torch.bfloat16)[0].contiguous())
    ys = {t: torch.empty(n, dtype=torch.float32, device=dev) for t, (p, s, n, k) in keep.items()}

    def run():
        for t, (p, s, n, k) in keep.items():
            tqa.gemv(p, s, xr[t], rotated=True, out=ys[t])

    ms = _time(torch, stream, run, 10)
    byts = sum(gemv_bytes(n, k) for (p, s, n, k) in keep.values())
    res["ffn_trio_gemv"] = {"packed_GB": round(sum(WEIGHT_BYTES_PER_ELEM * n * k for (_, _, n, k) in keep.values()) / 1e9, 3),
                            "us": round(ms * 1e3, 1), "GB_s": round(byts / (ms * 1e-3) / 1e9, 1)}
    return res


def cpu_baseline(model, groups, seconds):
    """The CPU oracle's float64 GEMV on sampled rows of the same packed weights, scaled to GB/s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import tq4_1s as otq

    rows = 256
    samples = []
    for it, gname in enumerate(list(groups) * 2):
        n, k = groups[gname]
        p, s = model[it % len(model)][gname]
        r0 = (it * 997) % (n - rows)
        x = np.random.default_rng(it).standard_normal(k).astype(np.float32)
        samples.append((p[r0:r0 + rows].cpu().numpy(), s[r0:r0 + rows].cpu().numpy().view(np.uint16), x, k))
    done_bytes = 0.0
    elapsed = 0.0
    it = 0
    while elapsed < seconds:
        pk, sc, x, k = samples[it % len(samples)]
        t = time.perf_counter()
        otq.gemv_rows_o64(pk, sc, x)
        elapsed += time.perf_counter() - t
        done_bytes += gemv_bytes(rows, k)
        it += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    # The same GEMV on one thread, and the float32 quantizer, on short samples.
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        st_bytes = st_time = 0.0
        j = 0
        while st_time < max(2.0, seconds / 6):
            pk, sc, x, k = samples[j % len(samples)]
            t = time.perf_counter()
            otq.gemv_rows_o64(pk, sc, x)
            st_time += time.perf_counter() - t
            st_bytes += gemv_bytes(rows, k)
            j += 1
    Wq = np.random.default_rng(7).standard_normal((rows, 4096)).astype(np.float32) * np.float32(4096 ** -0.5)
    q_time = q_weights = 0.0
    while q_time < 2.0:
        t = time.perf_counter()
        otq.quantize_o32(Wq)
        q_time += time.perf_counter() - t
        q_weights += Wq.size
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{it} oracle float64 GEMV calls on {rows}-row slices of the 8B decode groups "
                      f"(q|k|v, o, gate|up, down; {elapsed:.1f} s of oracle time)",
            "host_cpus": len(os.sched_getaffinity(0)),
            "single_thread_GB_s": round(st_bytes / st_time / 1e9, 4),
            "quantize_GB_s": round(q_weights * (4 + WEIGHT_BYTES_PER_ELEM) / q_time / 1e9, 4),
            "quantize_sample": f"oracle float32 quantizer on a {rows} x 4096 float32 matrix, {q_time:.1f} s"}


if __name__ == "__main__":
    main()
