"""rocprofv3 summaries of the decode GEMV: HBM traffic and kernel durations.

HBM traffic, from the repository root:

    rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o fetch -- python3 -m dequant_gemv_tq_amd.profiling run
    rocprofv3 --pmc WRITE_SIZE -d OUT/write -o write -- python3 -m dequant_gemv_tq_amd.profiling run
    python3 -m dequant_gemv_tq_amd.profiling summarize OUT/fetch/fetch_results.db OUT/write/write_results.db \\
        > profiles/gemv_traffic_llama8b.md

MFMA utilisation of the small-batch GEMM:

    rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 -d OUT/mfma -o mfma -- python3 -m dequant_gemv_tq_amd.profiling gemm_run
    python3 -m dequant_gemv_tq_amd.profiling gemm_summarize OUT/mfma/mfma_results.db > profiles/...md

HBM traffic of the turbo4 KV-cache decode attention (``kv_run`` / ``kv_summarize``, same pattern).

Kernel durations of a benchmark run:

    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o bench -- \\
        python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline
    python3 -m dequant_gemv_tq_amd.profiling stats OUT/trace/bench_kernel_stats.csv > profiles/...md
    python3 -m dequant_gemv_tq_amd.profiling groups OUT/trace/bench_kernel_trace.csv > profiles/...md

``groups`` takes the same run's kernel trace: the duration of every GEMV of the
graph-replayed decode steps by group, against the plain-read kernel over the
same bytes (the benchmark's read envelope, launched in group order).

``run`` launches, in this order: a plain elementwise copy (negation) of
1 GiB (calibration: it reads and writes exactly 1 GiB), then for each Llama-3-8B decode group
(q|k|v, o, gate|up, down) eight fused GEMVs over eight distinct copies of one
quantized layer with a bf16 activation.  ``summarize`` reads the two
counter databases, turns the KiB per dispatch of each counter into bytes with
the factor the copy kernel gives (known bytes / counted bytes) and writes a
short Markdown summary ending in one JSON line that the benchmark reads.  The
JSON carries the SHA-256 of the GEMV sources, so that a number taken before a
kernel change is not reported for the changed kernel.
"""

from __future__ import annotations

import hashlib
import json
import os
import sqlite3
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
GROUPS = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096), "down": (4096, 14336)}
MEMBERS = {"qkv": ["q", "k", "v"], "o": ["o"], "gate_up": ["gate", "up"], "down": ["down"]}
COPIES = 8
COPY_BYTES = 1 << 30
DOMINANT = ("qkv", "o", "gate_up")          # groups served by the dominant instantiation
DOMINANT_KERNEL = "gemv_kernel<FmtTQ4, 1, 1, 1, 3, 1024, 2, 1, 1>"   # K = 4096, one row per wavefront
GATE_UP_70B_KERNEL = "gemv_kernel<FmtTQ4, 1, 1, 1, 3, 1024, 2, 1, 2>"  # K = 8192 (Llama-3-70B gate|up in the benchmark)
SOURCES = ("csrc/tq_gemv.hip", "csrc/tq_internal.hpp")


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic_bytes(n: int, k: int, x_bytes: int = 2) -> int:
    """Packed nibbles + fp16 scales + activation + fp32 output of one GEMV."""
    return n * k // 2 + n * k // 16 * 2 + k * x_bytes + n * 4


def run() -> None:
    sys.path.insert(0, ROOT)
    import torch
    import dequant_gemv_tq_amd as tqa
    import workloads as wl

    dev = torch.device("cuda:0")
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)             # an elementwise kernel (copy_ may become a DMA transfer)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()
    for gname, (n, k) in GROUPS.items():
        W = torch.cat([wl.llama8b_weight(t, 0, dev) for t in MEMBERS[gname]], dim=0)
        p, s = tqa.quantize(W)
        del W
        reps = [(p.clone(), s.clone()) for _ in range(COPIES)]
        x = wl.activation(1, k, wl.generator(wl.seed_of(2, 0, 50), dev), dev, torch.bfloat16)[0].contiguous()
        y = torch.empty(n, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for pp, ss in reps:
            tqa.gemv(pp, ss, x, out=y)
        torch.cuda.synchronize()
        del reps, p, s
        torch.cuda.empty_cache()
    print("traffic run done", flush=True)


GEMM_BATCHES = (16, 32, 64)


def gemm_run() -> None:
    """Small-batch GEMM over one Llama-3-8B layer's groups at M = 16, 32, 64 (bf16 pre-rotated activations),
    COPIES launches per group and batch, for the MFMA counters."""
    sys.path.insert(0, ROOT)
    import torch
    import dequant_gemv_tq_amd as tqa
    import workloads as wl

    dev = torch.device("cuda:0")
    for gname, (n, k) in GROUPS.items():
        W = torch.cat([wl.llama8b_weight(t, 0, dev) for t in MEMBERS[gname]], dim=0)
        p, s = tqa.quantize(W)
        del W
        for m in GEMM_BATCHES:
            X = tqa.rotate(wl.activation(m, k, wl.generator(wl.seed_of(3, m, 0), dev), dev, torch.bfloat16),
                           dtype=torch.bfloat16)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            for _ in range(COPIES):
                tqa.gemm(p, s, X, out=y)
            torch.cuda.synchronize()
    print("gemm counter run done", flush=True)


GEMM_SQ = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_ANY",
           "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES")


def _gemm_dispatches(db: str, counters) -> list:
    con = sqlite3.connect(db)
    marks = ", ".join("?" for _ in counters)
    rows = con.execute(
        "select dispatch_id, kernel_name, counter_name, sum(value) from counters_collection "
        f"where counter_name in ({marks}) group by dispatch_id, kernel_name, counter_name "
        "order by dispatch_id", tuple(counters)).fetchall()
    con.close()
    per = {}
    for d, name, cname, v in rows:
        if "gemm_small_kernel" not in name:
            continue
        per.setdefault(d, {"name": name})[cname] = v
    disp = [per[d] for d in sorted(per)]
    expect = len(GROUPS) * len(GEMM_BATCHES) * COPIES
    if len(disp) != expect:
        raise RuntimeError(f"expected {expect} GEMM dispatches, found {len(disp)}")
    return disp


def gemm_summarize(db: str, sq_db: str | None = None) -> None:
    """MFMA utilisation and bf16 MFMA flops per GEMM dispatch from a --pmc MfmaUtil MfmaFlopsBF16 run, and
    (with a second database from a --pmc run of GEMM_SQ) the wavefronts' instruction counts and waits."""
    disp = _gemm_dispatches(db, ("MfmaUtil", "MfmaFlopsBF16"))
    lines = ["# Small-batch GEMM: MFMA utilisation (Llama-3-8B groups, bf16 pre-rotated activations)", "",
             "Commands (repository root on the GPU host; OUT is any scratch folder):", "", "```",
             "rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 -d OUT/mfma -o mfma -- python3 -m dequant_gemv_tq_amd.profiling "
             "gemm_run",
             "rocprofv3 --pmc " + " ".join(GEMM_SQ) + " -d OUT/sq -o sq -- python3 -m "
             "dequant_gemv_tq_amd.profiling gemm_run",
             "python3 -m dequant_gemv_tq_amd.profiling gemm_summarize OUT/mfma/mfma_results.db OUT/sq/sq_results.db",
             "```", "",
             "MfmaUtil is rocprofv3's derived counter (MFMA busy cycles over GPU-active cycles times SIMD count, "
             "in %); MfmaFlopsBF16 counts the bf16 MFMA work issued, against 2 * 16 * ceil(M / 16) * N * K for "
             "the padded activation tiles.", "",
             "| group | N x K | M | kernel | MFMA busy % | bf16 MFMA GFLOP per launch | padded 2*M*N*K GFLOP |",
             "|---|---|---|---|---|---|---|"]
    i = 0
    for gname, (n, k) in GROUPS.items():
        for m in GEMM_BATCHES:
            chunk = disp[i:i + COPIES]
            i += COPIES
            util = statistics.median(c.get("MfmaUtil", 0.0) for c in chunk)
            fl = statistics.median(c.get("MfmaFlopsBF16", 0.0) for c in chunk)
            import re
            kn = re.search(r"gemm_small_kernel<[^>]*>", chunk[0]["name"].replace("tq::(anonymous namespace)::", ""))
            lines.append(f"| {gname} | {n} x {k} | {m} | `{kn.group(0) if kn else chunk[0]['name']}` | {util:.1f} | "
                         f"{fl / 1e9:.3f} | {2 * 16 * ((m + 15) // 16) * n * k / 1e9:.3f} |")
    if sq_db:
        sq = _gemm_dispatches(sq_db, GEMM_SQ)
        lines += ["", "Wavefront counters (median over the launches; SQ_WAVE_CYCLES is the summed lifetime of the "
                  "wavefronts, so the wait columns are shares of it):", "",
                  "| group | M | VALU instr per wavefront | LDS instr per wavefront | waiting (SQ_WAIT_ANY) % | "
                  "waiting on LDS (SQ_WAIT_INST_LDS) % | issuing VALU (SQ_ACTIVE_INST_VALU) % |",
                  "|---|---|---|---|---|---|---|"]
        i = 0
        for gname, (n, k) in GROUPS.items():
            for m in GEMM_BATCHES:
                chunk = sq[i:i + COPIES]
                i += COPIES

                def med(key, chunk=chunk):
                    return statistics.median(c.get(key, 0.0) for c in chunk)
                waves, cyc = max(med("SQ_WAVES"), 1.0), max(med("SQ_WAVE_CYCLES"), 1.0)
                lines.append(f"| {gname} | {m} | {med('SQ_INSTS_VALU') / waves:.0f} | "
                             f"{med('SQ_INSTS_LDS') / waves:.0f} | {100 * med('SQ_WAIT_ANY') / cyc:.1f} | "
                             f"{100 * med('SQ_WAIT_INST_LDS') / cyc:.1f} | "
                             f"{100 * med('SQ_ACTIVE_INST_VALU') / cyc:.1f} |")
    print("\n".join(lines + [""]))


def _per_dispatch(db: str, counter: str):
    con = sqlite3.connect(db)
    rows = con.execute(
        "select dispatch_id, kernel_name, sum(value) from counters_collection where counter_name = ? "
        "group by dispatch_id, kernel_name order by dispatch_id", (counter,)).fetchall()
    con.close()
    return [(d, name, v) for d, name, v in rows]


def _split(rows):
    copies = [v for _, name, v in rows if "neg_kernel" in name]
    gemv = [(name, v) for _, name, v in rows if "gemv_kernel" in name]
    if len(gemv) != COPIES * len(GROUPS):
        raise RuntimeError(f"expected {COPIES * len(GROUPS)} GEMV dispatches, found {len(gemv)}")
    per = {}
    for i, gname in enumerate(GROUPS):
        chunk = gemv[i * COPIES:(i + 1) * COPIES]
        per[gname] = (chunk[0][0], statistics.median(v for _, v in chunk))
    if not copies:
        raise RuntimeError("calibration copy (negation kernel) not found")
    return statistics.median(copies), per


def summarize(fetch_db: str, write_db: str) -> None:
    f_copy, f_per = _split(_per_dispatch(fetch_db, "FETCH_SIZE"))
    w_copy, w_per = _split(_per_dispatch(write_db, "WRITE_SIZE"))
    kib = COPY_BYTES / 1024
    f_scale = kib / f_copy
    w_scale = kib / w_copy
    lines = [
        "# Decode GEMV HBM traffic (Llama-3-8B groups, bf16 activation, fused rotation)",
        "",
        "Commands (repository root on the GPU host; OUT is any scratch folder):",
        "",
        "```",
        "rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o fetch -- python3 -m dequant_gemv_tq_amd.profiling run",
        "rocprofv3 --pmc WRITE_SIZE -d OUT/write -o write -- python3 -m dequant_gemv_tq_amd.profiling run",
        "python3 -m dequant_gemv_tq_amd.profiling summarize OUT/fetch/fetch_results.db OUT/write/write_results.db",
        "```",
        "",
        f"Calibration: a 1 GiB elementwise copy reads FETCH_SIZE = {f_copy:.0f} KiB and WRITE_SIZE = {w_copy:.0f} KiB "
        f"per dispatch; scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write) turn counted KiB into bytes.",
        "",
        "| group | N x K | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic MB (scaled) | algorithmic MB | ratio |",
        "|---|---|---|---|---|---|---|",
    ]
    dom_t = dom_a = 0.0
    for gname, (n, k) in GROUPS.items():
        fk = f_per[gname][1]
        wk = w_per[gname][1]
        t = (fk * f_scale + wk * w_scale) * 1024
        alg = algorithmic_bytes(n, k)
        if gname in DOMINANT:
            dom_t += t
            dom_a += alg
        lines.append(f"| {gname} | {n} x {k} | {fk:.0f} | {wk:.0f} | {t / 1e6:.2f} | {alg / 1e6:.2f} | {t / alg:.3f} |")
    rec = {"kernel": DOMINANT_KERNEL, "groups": list(DOMINANT),
           "traffic_bytes_per_launch": round(dom_t / len(DOMINANT)),
           "algorithmic_bytes_per_launch": round(dom_a / len(DOMINANT)),
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "source_sha256": source_hash()}
    lines += ["", "Per launch of the dominant instantiation (mean over q|k|v, o and gate|up):", "",
              f"traffic-json: {json.dumps(rec)}", ""]
    print("\n".join(lines))


# turbo4 KV-cache decode attention: the Llama-3-8B head layout, 16 sequences x 4096 cached tokens, four layers
# with distinct caches (424 MB together, more than the 256 MB Infinity Cache).
KV_LAYOUT = {"batch": 16, "context": 4096, "q_heads": 32, "kv_heads": 8, "head_dim": 128, "layers": 4}
KV_BYTES_PER_TOKEN_HEAD = 128 + 8 + 64 + 2


def kv_run() -> None:
    sys.path.insert(0, ROOT)
    import torch
    import dequant_gemv_tq_amd as tqa
    import workloads as wl

    dev = torch.device("cuda:0")
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()
    L = KV_LAYOUT
    B, T, Hq, Hkv, D = L["batch"], L["context"], L["q_heads"], L["kv_heads"], L["head_dim"]
    caches = []
    for layer in range(L["layers"]):
        g = wl.generator(wl.seed_of(6, layer, 0), dev)
        K = torch.randn((B, Hkv, T, D), generator=g, device=dev).to(torch.bfloat16)
        V = torch.randn((B, Hkv, T, D), generator=g, device=dev).to(torch.bfloat16)
        caches.append(tqa.kv_quantize_k(K) + tqa.kv_quantize_v(V))
        del K, V
    torch.cuda.empty_cache()
    q = torch.randn((B, Hq, D), generator=wl.generator(wl.seed_of(6, 99, 1), dev), device=dev).to(torch.bfloat16)
    lengths = torch.full((B,), T, dtype=torch.int32, device=dev)
    o = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(tqa.attn_workspace_bytes(B, Hq, T), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for kc, ks, vp, vn in caches:
        tqa.attn_decode(q, lengths, kc, ks, vp, vn, out=o, workspace=ws)
    torch.cuda.synchronize()
    print("kv traffic run done", flush=True)


def kv_summarize(fetch_db: str, write_db: str) -> None:
    def split(rows):
        copies = [v for _, name, v in rows if "neg_kernel" in name]
        att = [(name, v) for _, name, v in rows if "attn_" in name]
        sp = [v for name, v in att if "attn_split_kernel" in name]
        cb = [v for name, v in att if "attn_combine_kernel" in name]
        if not copies or len(sp) != KV_LAYOUT["layers"] or len(cb) != KV_LAYOUT["layers"]:
            raise RuntimeError("unexpected dispatches in the KV counter run")
        return statistics.median(copies), statistics.median(sp), statistics.median(cb)

    fc, fs, fcb = split(_per_dispatch(fetch_db, "FETCH_SIZE"))
    wc, ws, wcb = split(_per_dispatch(write_db, "WRITE_SIZE"))
    kib = COPY_BYTES / 1024
    f_scale, w_scale = kib / fc, kib / wc
    L = KV_LAYOUT
    B, T, Hq, Hkv, D = L["batch"], L["context"], L["q_heads"], L["kv_heads"], L["head_dim"]
    cache = B * T * Hkv * KV_BYTES_PER_TOKEN_HEAD
    alg = cache + B * Hq * D * (2 + 4)
    splits = (T + 255) // 256
    partials = B * Hq * splits * (D + 2) * 4
    t_split = (fs * f_scale + ws * w_scale) * 1024
    t_comb = (fcb * f_scale + wcb * w_scale) * 1024
    lines = [
        "# turbo4 KV-cache decode attention: HBM traffic (Llama-3-8B heads, 16 sequences x 4096 tokens)",
        "",
        "Commands (repository root on the GPU host; OUT is any scratch folder):",
        "",
        "```",
        "rocprofv3 --pmc FETCH_SIZE -d OUT/kvf -o kvf -- python3 -m dequant_gemv_tq_amd.profiling kv_run",
        "rocprofv3 --pmc WRITE_SIZE -d OUT/kvw -o kvw -- python3 -m dequant_gemv_tq_amd.profiling kv_run",
        "python3 -m dequant_gemv_tq_amd.profiling kv_summarize OUT/kvf/kvf_results.db OUT/kvw/kvw_results.db",
        "```",
        "",
        f"Calibration as for the GEMV: a 1 GiB elementwise copy reads FETCH_SIZE = {fc:.0f} KiB and WRITE_SIZE = "
        f"{wc:.0f} KiB; scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write).",
        "",
        "| kernel (per layer, median of 4) | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic MB (scaled) |",
        "|---|---|---|---|",
        f"| `attn_split_kernel<4, bf16 q>` | {fs:.0f} | {ws:.0f} | {t_split / 1e6:.2f} |",
        f"| `attn_combine_kernel` | {fcb:.0f} | {wcb:.0f} | {t_comb / 1e6:.2f} |",
        "",
        f"Algorithmic bytes per layer: the quantized cache {cache / 1e6:.2f} MB ({KV_BYTES_PER_TOKEN_HEAD} B per token "
        f"and cache head) plus q and o, {alg / 1e6:.2f} MB; the split partials (m, l, z per sequence, head and "
        f"256-token split) add {partials / 1e6:.2f} MB written and read back by design.  Measured / algorithmic: "
        f"{(t_split + t_comb) / alg:.3f} (split + combine), {(t_split + t_comb) / (alg + 2 * partials):.3f} with the "
        "partials counted.",
        "",
    ]
    print("\n".join(lines))


TRACE_COMMAND = ("rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o bench -- "
                 "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline")
STATS_SOURCES = ("csrc/tq_gemv.hip", "csrc/tq_internal.hpp", "csrc/tq_gemm.hip", "csrc/tq_blockfp.hip",
                 "csrc/tq_transform.hip", "csrc/tq_q8.hip", "csrc/tq_kv.hip", "csrc/tq_measure.hip")


def stats_source_hash() -> str:
    h = hashlib.sha256()
    for rel in STATS_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stats(csv_path: str) -> None:
    """Markdown table of the library's kernels from a rocprofv3 kernel_stats.csv."""
    import csv
    import re
    rows = list(csv.DictReader(open(csv_path)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    averages = {}
    lines = ["# Kernel durations of the benchmark (Llama-3-8B decode stream and secondary rows)", "",
             "Command (repository root on the GPU host; OUT is any scratch folder):", "", "```",
             TRACE_COMMAND, "python3 -m dequant_gemv_tq_amd.profiling stats OUT/trace/bench_kernel_stats.csv",
             "```", "",
             "Library kernels (`tq::`), from rocprofv3's kernel statistics; durations in microseconds.", "",
             "| kernel | calls | average | min | max | share of all GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        m = re.search(r"tq::\(anonymous namespace\)::(\w+(?:<[^>]*>)?)", r["Name"])
        if not m:
            continue
        name = m.group(1).replace("tq::(anonymous namespace)::", "")
        averages[name] = round(float(r["AverageNs"]) / 1e3, 3)
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.2f}% |")
    lines += ["", "Decode GEMV instantiations `gemv_kernel<format, J, R, MC, mode, threads, depth, early, stage>`: "
              "q|k|v, o and gate|up (K = 4096, bf16 activation, rotation fused, one row per wavefront) run "
              f"`{DOMINANT_KERNEL}`; down "
              "(K = 14336, two row slots per workgroup) rotates its activation per lane, `gemv_kernel<FmtTQ4, 1, 1, 1, 3, 1024, 2, 1, 0>`.  "
              "Other kernels: the quantizer (`quantize_kernel<bf16, rsf>`, the second flag for the RSF-lite "
              "scale search), the small-batch GEMM (VALU `gemv_kernel<..., MC, ...>` for M <= 2, and float32 "
              "activations below 16 rows; above, the persistent MFMA `gemm_small_kernel<format, MT, NQ>` with bf16 "
              "activations, MT = 1, 2, 4 "
              "tiles of 16 activation rows, and `gemm_mfma_kernel` with float32 activations), dequantization, "
              "the NVFP4 / MXFP6 rows (`gemv_kernel<FmtNVFP4, ...>`, `gemv_kernel<FmtMXFP6, ...>` up to four "
              "activation rows, `gemm_small_kernel<GemmNVFP4, ...>`, `gemm_small_kernel<GemmMXFP6, ...>` from "
              "three) and the "
              "load-time int8 rows (`q8_transcode_kernel`, `q8_gemv_kernel<bf16 activation, passes>`), the turbo4 KV "
              "cache (`q8_rows_kernel` keys, `turbo4_encode_kernel` values, `attn_split_kernel<G, bf16 q>` + "
              "`attn_combine_kernel` for decode attention), `stream_read_kernel` (the read envelope); the "
              "remaining GPU time is PyTorch drawing the synthetic weights.", "",
              "Average durations (microseconds) as the benchmark reads them:", "",
              "stats-json: " + json.dumps({"kernels": averages, "source_sha256": stats_source_hash()}), ""]
    print("\n".join(lines))


def read_stats_record(path: str) -> dict | None:
    """The kernel averages of a stats summary, or None when absent or taken from other sources."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("stats-json: "):
                    rec = json.loads(line[len("stats-json: "):])
                    return rec if rec.get("source_sha256") == stats_source_hash() else None
    except OSError:
        return None
    return None


def read_record(path: str) -> dict | None:
    """The JSON line of a summary, or None when absent or taken from other sources."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    return rec if rec.get("source_sha256") == source_hash() else None
    except OSError:
        return None
    return None


DOWN_KERNEL = "gemv_kernel<FmtTQ4, 1, 1, 1, 3, 1024, 2, 1, 0>"   # K = 14336, activation rotated per lane


def groups(csv_path: str) -> None:
    """Per-group GEMV kernel durations of the decode steps in a rocprofv3 kernel trace, and the plain read."""
    import csv
    import re
    rows = []
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if "tq::" not in r["Kernel_Name"]:
                continue                   # the library's kernels only (not PyTorch's input generation)
            name = r["Kernel_Name"].replace("tq::(anonymous namespace)::", "")
            m = re.search(r"([A-Za-z0-9_]+(<[^()]*>)?)\(", name)
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), m.group(1) if m else name))
    rows.sort()
    names = [r[2] for r in rows]
    order = list(GROUPS)
    kern = {"qkv": DOMINANT_KERNEL, "o": DOMINANT_KERNEL, "gate_up": DOMINANT_KERNEL, "down": DOWN_KERNEL}
    layer = [kern[g] for g in order]
    # A decode step: 32 layers of the four group launches back to back.
    step = layer * 32
    per = {g: [] for g in order}
    spans = []
    i = 0
    while i + len(step) <= len(rows):
        if names[i:i + len(step)] == step:
            for j in range(len(step)):
                per[order[j % 4]].append((rows[i + j][1] - rows[i + j][0]) / 1e3)
            spans.append((rows[i + len(step) - 1][1] - rows[i][0]) / 1e3)
            i += len(step)
        else:
            i += 1
    # The read envelope: runs of consecutive plain reads, one run per group in group order.
    reads, run = [], []
    for k, n in enumerate(names):
        if n == "stream_read_kernel":
            if run and k != run[-1] + 1:
                reads.append(run)
                run = []
            run.append(k)
    if run:
        reads.append(run)
    env = {}
    if len(reads) == len(order):
        for g, r in zip(order, reads):
            env[g] = statistics.median((rows[k][1] - rows[k][0]) / 1e3 for k in r)
    lines = ["# Decode GEMV durations by group (Llama-3-8B layer shapes, rocprofv3 kernel trace)", "",
             "Command (repository root on the GPU host; OUT is any scratch folder):", "", "```",
             "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o bench -- "
             "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline",
             "python3 -m dequant_gemv_tq_amd.profiling groups OUT/trace/bench_kernel_trace.csv", "```", "",
             f"{len(spans)} graph-replayed decode steps of 128 launches found in the trace (the first replays "
             "include the profiler's warm-up). Kernel execution time per launch, median over every layer of "
             "every step; the plain read is `stream_read_kernel` over the same bytes with the same launch "
             "shape (the benchmark's read envelope).", "",
             "| group | N x K | kernel | GEMV median us | plain read median us | GEMV / read |",
             "|---|---|---|---|---|---|"]
    rec = {}
    for g in order:
        n, k = GROUPS[g]
        gm = statistics.median(per[g]) if per[g] else float("nan")
        rm = env.get(g, float("nan"))
        rec[g] = {"gemv_us": round(gm, 2), "read_us": round(rm, 2), "ratio": round(gm / rm, 3)}
        lines.append(f"| {g} | {n} x {k} | `{kern[g]}` | {gm:.2f} | {rm:.2f} | {gm / rm:.3f} |")
    if spans:
        lines += ["", f"Step span (first launch start to last launch end), median: {statistics.median(spans):.1f} us.",
                  ""]
    lines += ["groups-json: " + json.dumps({"groups": rec, "source_sha256": stats_source_hash()}), ""]
    print("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) == 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    elif len(sys.argv) == 3 and sys.argv[1] == "stats":
        stats(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "groups":
        groups(sys.argv[2])
    elif len(sys.argv) >= 2 and sys.argv[1] == "gemm_run":
        gemm_run()
    elif len(sys.argv) in (3, 4) and sys.argv[1] == "gemm_summarize":
        gemm_summarize(sys.argv[2], sys.argv[3] if len(sys.argv) == 4 else None)
    elif len(sys.argv) >= 2 and sys.argv[1] == "kv_run":
        kv_run()
    elif len(sys.argv) == 4 and sys.argv[1] == "kv_summarize":
        kv_summarize(sys.argv[2], sys.argv[3])
    else:
        print(__doc__)
        sys.exit(2)
