#!/usr/bin/env python3
"""Decode benchmark of compressed-KV attention (DepthWeave-KV) on one MI355X.

A step is one decode token for every sequence: for each layer, decode
attention over the whole compressed cache, then the append of the new
token's K/V (the attend-then-append order of the decode procedure).  Inputs
(cache, queries, new tokens) are resident in HBM before timing; steps are
replayed from HIP graphs captured in chunks.  Prints one JSON line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workload as w  # noqa: E402
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases, max_tier_counts  # noqa: E402

METRIC = "decode tokens/s + achieved HBM GB/s (% of peak), compressed-KV attn at 64K"
PEAK_HBM_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# every file the decode kernel's translation units read (the kernel, its
# instances, the append encoder compiled into the one-launch step, the shared
# device helpers and declarations, the layout, the C header) and the build
# flags it is compiled with
_CSRC = os.path.join(ROOT, "compressed_kv_cache_dwkv_amd", "csrc")
_SHARED_SRCS = [os.path.join(_CSRC, f) for f in ("device.h", "kernels.h", "layout.h")] + \
               [os.path.join(ROOT, "include", "dwkv.h"), os.path.join(ROOT, "compressed_kv_cache_dwkv_amd", "build.py")]
DECODE_SRCS = [os.path.join(_CSRC, f) for f in ("decode_impl.h", "decode.hip", "decode8.hip", "append_body.h")] + \
              _SHARED_SRCS


def decode_source_sha() -> str:
    """sha256 of the decode kernel's sources: every file its translation
    units include and the build flags it is compiled with."""
    h = hashlib.sha256()
    for f in DECODE_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def workload_name(cfg) -> str:
    return cfg.name if cfg.coef_bits == 16 else cfg.name + "-int8coef"


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's)")
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--config", type=int, default=2, help="workload index 0-4 (2 = 64K headline)")
    p.add_argument("--chunk", type=int, default=16, help="steps per captured graph")
    p.add_argument("--splits", type=int, default=0, help="decode workgroups per KV head (0 = auto)")
    p.add_argument("--context", type=int, default=0,
                   help="tokens already cached per sequence in place of the workload's (0 = the workload's); "
                        "the workload is then named with the context, so no recorded counter traffic applies")
    p.add_argument("--batch", type=int, default=0,
                   help="sequences per step in place of the workload's (0 = the workload's); the workload is "
                        "then named with the batch, so no recorded counter traffic applies to it")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    p.add_argument("--kernel-reps", type=int, default=10)
    p.add_argument("--separate", action="store_true",
                   help="two launches per layer (dwkv_decode_attn, dwkv_append) instead of dwkv_decode_step")
    p.add_argument("--comparator", choices=["dense", "unfused"], default=None,
                   help="time a comparator instead of the fused step: 'dense' = flash-decode over a dense fp16 "
                        "cache of the same shape; 'unfused' = per layer, materialise K^/V^ to HBM, dense "
                        "flash-decode over it, then the append")
    p.add_argument("--coef-bits", type=int, choices=[8, 16], default=16,
                   help="coefficient form: 16 = fp16, 8 = the 8-bit blockwise form (int8 codes, fp16 block scales)")
    p.add_argument("--dense-splits", type=int, default=0, help="dense decode workgroups per KV head (0 = auto)")
    p.add_argument("--stream-probe", action="store_true",
                   help="time a plain streaming read of one decode launch's algorithmic bytes per layer, "
                        "launched like the decode (graph replays over the layers), at several grids")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 512 MiB device copy (counter calibration)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                        "script with --copy-probe into profiles/ and exit")
    p.add_argument("--trace-summary", metavar="TRACE_DIR",
                   help="summarise a rocprofv3 --kernel-trace --stats run of this script into "
                        "profiles/ and exit")
    p.add_argument("--mode", choices=["decode", "prefill"], default="decode",
                   help="decode: the decode step (the headline); prefill: compression of the workload's "
                        "prompt into the cache (Gram sums, bases, bulk encode for every layer)")
    p.add_argument("--power-iters", type=int, default=2, help="prefill: range-finder power iterations")
    p.add_argument("--bench-json", metavar="FILE",
                   help="a run's saved stdout, whose last JSON line is used: with --trace-summary, a default "
                        "run of the same build, quoted beside the trace; with --pmc-summary, the counter run's "
                        "own output (its algorithmic bytes per launch)")
    return p.parse_args()


COPY_PROBE_BYTES = 512 << 20


def _pmc_per_dispatch(run_dir: str, counter: str):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            key = (row["Kernel_Name"], row["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def _json_line(path: str) -> dict:
    """The last JSON object line of a file (a bench run's output, possibly
    mixed with a profiler's messages)."""
    lines = [l for l in open(path).read().splitlines() if l.startswith("{")]
    return json.loads(lines[-1])


def pmc_summary(workload: str, fetch_dir: str, write_dir: str, bench_json: Optional[str] = None):
    """HBM bytes per decode launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy
    of COPY_PROBE_BYTES bytes in the same process."""
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _pmc_per_dispatch(d, counter)
        dec = [v for k, vs in per.items() if "decode_kernel" in k for v in vs]
        cpy = [v for k, vs in per.items() if ("copyBuffer" in k or "copy" in k.lower()) and "decode" not in k
               for v in vs]
        cpy = [v for v in cpy if v * 1024 > COPY_PROBE_BYTES / 4]          # the probe, not small copies
        if not dec or not cpy:
            raise SystemExit(f"{counter}: decode dispatches {len(dec)}, copy-probe dispatches {len(cpy)}")
        scale = COPY_PROBE_BYTES / (float(np.mean(cpy)) * 1024)
        res[counter] = {"decode_kib_mean": float(np.mean(dec)), "decode_dispatches": len(dec),
                        "copy_kib_mean": float(np.mean(cpy)), "copy_dispatches": len(cpy),
                        "scale": scale, "bytes_per_launch": float(np.mean(dec)) * 1024 * scale}
    total = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    rec = {"workload": workload, "kernel": "decode_kernel",
           "decode_source_sha256": decode_source_sha(),
           "hbm_bytes_per_launch": total, "counters": res,
           "copy_probe_bytes": COPY_PROBE_BYTES}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.json")
    json.dump(rec, open(path, "w"), indent=1)
    base = workload[:-len("-int8coef")] if workload.endswith("-int8coef") else workload
    cfg = next(c for c in w.CONFIGS if c.name == base)
    ci = w.CONFIGS.index(cfg)
    cflag = " --coef-bits 8" if workload != base else ""
    alg = None
    if bench_json:     # the JSON line the counter run itself printed
        alg = _json_line(bench_json)["roofline"]["algorithmic_bytes_per_launch"]
        rec["algorithmic_bytes_per_launch"] = alg
        json.dump(rec, open(path, "w"), indent=1)
    f, wr = res["FETCH_SIZE"], res["WRITE_SIZE"]
    lines = [
        f"# decode_kernel HBM traffic, {workload}",
        "",
        "The kernel measured is the one-launch decode step (decode attention plus the append of the new",
        "token), as `bench.py` launches it.",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp on one MI355X), then the summary on any host:",
        "",
        "```",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o run -- python3 <repo>/bench.py "
        f"--config {ci}{cflag} {PMC_RUN_ARGS}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o run -- python3 <repo>/bench.py "
        f"--config {ci}{cflag} {PMC_RUN_ARGS}",
        f"python3 <repo>/bench.py --config {ci}{cflag} --pmc-summary <fetch> <write> --bench-json <fetch run's stdout file>",
        "```",
        "",
        "`--copy-probe` adds a plain 512 MiB device-to-device copy to the same process; each counter is",
        "scaled by (512 MiB) / (what the counter reads for that copy).",
        "",
        "| counter | decode KiB / dispatch (mean) | dispatches | copy KiB / dispatch | scale | decode bytes / launch |",
        "|---|---|---|---|---|---|",
        f"| FETCH_SIZE | {f['decode_kib_mean']:.1f} | {f['decode_dispatches']} | {f['copy_kib_mean']:.1f} | "
        f"{f['scale']:.4f} | {f['bytes_per_launch']:.0f} |",
        f"| WRITE_SIZE | {wr['decode_kib_mean']:.1f} | {wr['decode_dispatches']} | {wr['copy_kib_mean']:.1f} | "
        f"{wr['scale']:.4f} | {wr['bytes_per_launch']:.0f} |",
        "",
        f"HBM traffic per launch: {total:.0f} bytes"
        + (f", {total / alg:.3f}x the {alg:.0f} algorithmic bytes (reads {f['bytes_per_launch'] / alg:.3f}x)."
           if alg else "."),
        "",
        f"Decode source sha256: `{rec['decode_source_sha256']}` (bench.py reports `traffic` only while "
        "the decode sources and build flags match it).",
    ]
    open(os.path.join(PROFILES, f"decode_{workload}_traffic.md"), "w").write("\n".join(lines) + "\n")
    print(json.dumps(rec), flush=True)


PMC_RUN_ARGS = "--steps 2 --warmup 1 --no-cpu-baseline --copy-probe --kernel-reps 1"
TRACE_RUN_ARGS = "--steps 16 --warmup 2 --no-cpu-baseline"


def trace_summary(cfg, ci: int, trace_dir: str, bench_json: Optional[str]):
    """profiles/decode_<workload>_kernel_trace.md from a rocprofv3
    --kernel-trace --stats run (its *_kernel_stats.csv)."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    dec = [r for r in rows if "decode_kernel" in r["Name"]]
    if not dec:
        raise SystemExit("no decode_kernel in the trace")
    bj = _json_line(bench_json) if bench_json else None
    lines = [
        f"# decode_kernel, {workload_name(cfg)} (batch {cfg.batch}, {cfg.num_layers} layers, {cfg.num_q_heads} q / "
        f"{cfg.num_kv_heads} KV heads, d {cfg.head_dim}, {cfg.n_tokens} tokens)",
        "",
        "The kernel is the one-launch decode step (`dwkv_decode_step`: decode attention plus the append of the new",
        "token), which is what `bench.py` launches per layer.",
        "",
        "Command (run from /tmp with TMPDIR=/tmp on one MI355X), then the summary on any host:",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o bench -- python3 <repo>/bench.py "
        f"--config {ci}{' --coef-bits 8' if cfg.coef_bits == 8 else ''} {TRACE_RUN_ARGS}",
        f"python3 <repo>/bench.py --config {ci}{' --coef-bits 8' if cfg.coef_bits == 8 else ''} --trace-summary <out> "
        f"[--bench-json <default run's stdout file>]",
        "```",
        "",
        "Kernel statistics (durations in ns; graph replays of the warm-up and timed steps plus the replays of",
        "the one-step timing graph):",
        "",
        "| kernel | calls | average ns | min ns | max ns | stddev ns |",
        "|---|---|---|---|---|---|",
    ]
    for r in dec:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | {float(r['MinNs']):.0f} | "
                     f"{float(r['MaxNs']):.0f} | {float(r.get('StdDev', 0) or 0):.0f} |")
    avg = sum(float(r["AverageNs"]) * int(r["Calls"]) for r in dec) / sum(int(r["Calls"]) for r in dec)
    lines.append("")
    if bj:
        rf = bj["roofline"]
        alg = rf["algorithmic_bytes_per_launch"]
        lines += [
            f"Algorithmic bytes per launch: {alg:.0f} -> {alg / avg:.0f} GB/s at the trace average "
            f"({alg / avg / PEAK_HBM_GBPS * 100:.1f}% of {PEAK_HBM_GBPS:.0f} GB/s).",
            "",
            f"The same build's default `bench.py --config {ci}` run: {bj['value']:.1f} tokens/s, "
            f"{rf['mean_launch_us']:.2f} us per launch over its timed region ({rf['achieved']:.0f} GB/s, "
            f"{rf['frac'] * 100:.1f}% of peak), {rf['one_step_graph_launch_us']:.2f} us from replays of a graph",
            "of one step's launches.  The trace's start-to-end durations of back-to-back kernels include each",
            "kernel's end, which overlaps the next kernel's start.",
        ]
    open(os.path.join(PROFILES, f"decode_{workload_name(cfg)}_kernel_trace.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def _gen_layer_job(args):
    ci, layer, coef_bits, batch, n = args
    return gen_layer(w.get_config(ci).with_(coef_bits=coef_bits, batch=batch, n_tokens=n), layer)


def algorithmic_layer_bytes(cfg, counts: np.ndarray, app_tier: Optional[np.ndarray] = None) -> int:
    """Bytes one layer's decode step must move, the one accounting used for
    every figure: every cached token at its tier's size (fp16 coefficients at
    the routed rank; per K and V a residual block of channel indices, packed
    codes and an fp16 scale), both bases of every KV head (once: every
    sequence shares them), and -- with an append -- the appended token of each
    (sequence, KV head) at its tier's size.  Queries, outputs, split partials
    and padding are not counted."""
    per_tok = np.array([w.compressed_bytes_per_token(r, s, cfg.resid_bits, cfg.coef_bits)
                        for r, s in zip(cfg.tier_rank, cfg.resid_per_tier)])
    tok = float((counts.reshape(-1, cfg.num_tiers) * per_tok[None, :]).sum())
    bases = 2 * cfg.num_kv_heads * cfg.r_max * cfg.head_dim * 2
    app = 0.0 if app_tier is None else float(per_tok[app_tier.reshape(-1).astype(np.int64)].sum())
    return int(tok + bases + app)


def stored_traffic(workload: str):
    """HBM bytes per decode launch measured by rocprofv3 counters, if the
    summary in profiles/ was taken on the current decode kernel source."""
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = decode_source_sha()
    if rec.get("decode_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_step_rate(cfg, bases, appends, budget_s: float, threads: int):
    """The oracle's decode + append, layer by layer over one step (each
    layer's synthetic input regenerated first, outside the timing), until
    the budget is spent; returns (seconds per full step, layers timed, s)."""
    import oracle
    dt = 0.0
    done = 0
    for layer in range(cfg.num_layers):
        m = layer // cfg.layers_per_group
        lay = gen_layer(cfg, layer)
        q = gen_query(cfg, layer)
        t0 = time.perf_counter()
        oracle.decode(cfg, lay, bases["K"][m], bases["V"][m], q, threads=threads)
        a = appends[0][layer]
        oracle.append_layer(cfg, bases["K"][m], bases["V"][m], a["k"], a["v"], a["tier"])
        dt += time.perf_counter() - t0
        done += 1
        if dt >= budget_s:
            break
    return dt / done * cfg.num_layers, done, dt


def cpu_baseline(cfg, bases, appends, budget_s: float):
    """The oracle timed on this host's cores (all it may use, then one
    thread), on a bounded sample of one step, scaled to a full step.  The
    oracle runs one (sequence, KV head) per thread, so it uses at most
    B x H_kv threads."""
    import oracle
    host = len(os.sched_getaffinity(0))
    threads = min(oracle.max_threads(), host)
    used = min(threads, cfg.batch * cfg.num_kv_heads)
    step_s, done, dt = _oracle_step_rate(cfg, bases, appends, budget_s, threads)
    step_1, done_1, dt_1 = _oracle_step_rate(cfg, bases, appends, budget_s / 2, 1)
    return {
        "value": cfg.batch / step_s, "unit": "tokens/s", "cores": used, "kind": "oracle",
        "host_cores": host, "cpu_model": _cpu_model(),
        "value_1_thread": cfg.batch / step_1,
        "sample": f"{done} of {cfg.num_layers} layers of one step (decode over all "
                  f"{cfg.n_tokens} tokens x {cfg.batch * cfg.num_kv_heads} KV heads + append) "
                  f"on {used} threads, {dt:.1f} s; 1 thread: {done_1} layers, {dt_1:.1f} s; "
                  f"each scaled to a full step",
    }


def _time_graph_steps(step, W: int, K: int, chunk: int):
    """W eager warm-up steps, then K steps replayed from graphs of `chunk`
    steps; returns the elapsed milliseconds of the K steps."""
    import torch
    for s in range(W):
        step(s)
    torch.cuda.synchronize()
    graphs = []
    for c0 in range(W, W + K, chunk):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(c0, min(c0 + chunk, W + K)):
                step(s)
        graphs.append(g)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for g in graphs:
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end)


def _graph_launch_ms(launches, reps: int):
    """Mean milliseconds of one launch: the launches in one graph, replayed."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launches()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def _dense_splits(args, cfg) -> int:
    if args.dense_splits > 0:
        return args.dense_splits
    return max(1, min(256, 1024 // (cfg.batch * cfg.num_kv_heads)))


def run_dense(args, cfg, K: int, W: int):
    """Flash-decode over a dense fp16 cache of the workload's shape (every
    layer, the workload's context), the uncompressed baseline."""
    import torch
    from compressed_kv_cache_dwkv_amd import dwkv_dense_decode, dwkv_dense_workspace_bytes
    torch.cuda.set_device(0)
    L, B, H, Hq, d, n = cfg.num_layers, cfg.batch, cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.n_tokens
    n_cap = (n + 63) // 64 * 64
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed)
    Kd = torch.randn((L, B, H, n_cap, d), generator=gen, dtype=torch.float16, device="cuda")
    Vd = torch.randn((L, B, H, n_cap // 16, d, 16), generator=gen, dtype=torch.float16, device="cuda")
    q = torch.from_numpy(np.stack([gen_query(cfg, l) for l in range(L)])).cuda()
    out = torch.empty((L, B, Hq, d), dtype=torch.float32, device="cuda")
    S = _dense_splits(args, cfg)
    ws = torch.zeros(dwkv_dense_workspace_bytes(B, Hq, H, d, S), dtype=torch.uint8, device="cuda")
    n_dev = torch.full((B, H), n, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    print(f"bench: dense cache resident ({(Kd.numel() + Vd.numel()) * 2 / 1e9:.2f} GB), splits {S}",
          file=sys.stderr, flush=True)

    def step(s):
        for l in range(L):
            dwkv_dense_decode(q[l], Kd[l], Vd[l], n_dev, out[l], ws, S, scale)

    elapsed_ms = _time_graph_steps(step, W, K, args.chunk)
    launch_ms = elapsed_ms / (K * L)
    one_step_ms = _graph_launch_ms(lambda: step(0), args.kernel_reps) / L
    layer_bytes = B * H * n * d * 2 * 2
    achieved = layer_bytes / (launch_ms * 1e-3) / 1e9
    return {
        "metric": METRIC + " [comparator: dense fp16 cache]",
        "value": B * K / (elapsed_ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": elapsed_ms / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16 MFMA operands, fp32 accumulate", "data": "synthetic",
        "config": {"workload": cfg.name, "comparator": "dense", "batch": B, "context": n, "layers": L,
                   "q_heads": Hq, "kv_heads": H, "head_dim": d, "dense_splits": S,
                   "storage": "fp16 K rows and fp16 V in 16-token blocks, no compression",
                   "note": "attention only; the dense cache's append (one 512-byte K and V row per KV head) "
                           "is not launched"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None, "kernel": "dense_decode_kernel",
                     "algorithmic_bytes_per_launch": layer_bytes, "mean_launch_us": launch_ms * 1e3,
                     "launch_time_from": "timed region", "one_step_graph_launch_us": one_step_ms * 1e3},
        "cpu_baseline": None,
    }


def run_stream_probe(args, cfg, K: int, W: int):
    """The bandwidth a single launch that only reads one decode launch's
    algorithmic bytes reaches: one buffer of that size per layer, read by
    dwkv_stream_probe with the decode's grid and with wider ones, the
    launches replayed from graphs exactly as the decode steps are."""
    import torch
    from compressed_kv_cache_dwkv_amd import dwkv_stream_probe
    torch.cuda.set_device(0)
    lay = gen_layer(cfg, 0)
    # layer 0's tier counts, with an appended token of tier 0 per (sequence, KV head)
    tiers, n_tok = np.asarray(lay["tier"]), np.asarray(lay["n_tokens"])
    counts = np.zeros((cfg.batch, cfg.num_kv_heads, cfg.num_tiers), np.int64)
    for b in range(cfg.batch):
        for h in range(cfg.num_kv_heads):
            counts[b, h] = np.bincount(tiers[b, h, :int(n_tok[b])], minlength=cfg.num_tiers)[:cfg.num_tiers]
    per_layer = algorithmic_layer_bytes(cfg, counts, np.zeros((cfg.batch, cfg.num_kv_heads), np.int64))
    nbytes = (per_layer + 15) // 16 * 16
    L = cfg.num_layers
    slab = torch.empty((L, nbytes), dtype=torch.uint8, device="cuda")
    slab.view(torch.int32).random_()             # arbitrary contents, written once
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = max(1, min(256, -(-cus // (cfg.batch * cfg.num_kv_heads))))   # the decode's plan
    grids = [(splits * cfg.batch * cfg.num_kv_heads, 512), (1024, 256), (2048, 256), (4096, 256)]
    rows = []
    for wg, th in grids:
        def step(s, wg=wg, th=th):
            for l in range(L):
                dwkv_stream_probe(slab[l], nbytes, wg, th, 0x9E3779B9, sink)
        elapsed_ms = _time_graph_steps(step, W, K, args.chunk)
        launch_us = elapsed_ms / (K * L) * 1e3
        gbps = nbytes / (launch_us * 1e-6) / 1e9
        rows.append({"workgroups": wg, "threads": th, "mean_launch_us": launch_us, "achieved": gbps,
                     "frac": gbps / PEAK_HBM_GBPS})
        print(f"bench: stream probe {wg} x {th}: {launch_us:.2f} us per launch, {gbps:.0f} GB/s",
              file=sys.stderr, flush=True)
    best = max(rows, key=lambda r: r["achieved"])
    return {
        "metric": "streaming read of one decode launch's algorithmic bytes per layer (measurement aid)",
        "value": best["achieved"], "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "higher_is_better": True, "data": "synthetic",
        "config": {"workload": cfg.name, "bytes_per_launch": nbytes, "layers": L,
                   "decode_grid": [grids[0][0], grids[0][1]], "launch": "graph replays, one launch per layer"},
        "grids": rows,
        "peak": PEAK_HBM_GBPS,
    }


PREFILL_METRIC = "prefill compression tokens/s (prompt tokens, all layers: Gram sums, bases, bulk encode)"


PREFILL_SRCS = [os.path.join(_CSRC, "prefill.hip")] + _SHARED_SRCS   # its includes and build flags too
PREFILL_RUN_ARGS = "--mode prefill --steps 1 --warmup 1 --no-cpu-baseline --copy-probe --kernel-reps 1"
PREFILL_TRACE_ARGS = "--mode prefill --steps 3 --warmup 1 --no-cpu-baseline --kernel-reps 2"
PREFILL_KERNELS = ("gram_kernel", "gram_reduce_kernel", "bases_kernel", "transpose_basis_kernel", "basis_copy_kernel",
                   "count_kernel", "place_kernel", "encode_kernel", "publish_kernel")


def prefill_source_sha() -> str:
    h = hashlib.sha256()
    for f in PREFILL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _prefill_name(name: str) -> Optional[str]:
    for k in PREFILL_KERNELS:
        if "::" + k in name or name.startswith(k) or (" " + k) in name or (k + "<") in name:
            return k
    return None


def prefill_pmc_summary(cfg, ci: int, fetch_dir: str, write_dir: str, bench_json: Optional[str]):
    """HBM bytes per launch of the prefill kernels from FETCH_SIZE /
    WRITE_SIZE, scaled as for the decode kernel by a plain copy's reading."""
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _pmc_per_dispatch(d, counter)
        cpy = [v for k, vs in per.items() if "copyBuffer" in k for v in vs]
        cpy = [v for v in cpy if v * 1024 > COPY_PROBE_BYTES / 4]
        if not cpy:
            raise SystemExit(f"{counter}: no copy-probe dispatch")
        scale = COPY_PROBE_BYTES / (float(np.mean(cpy)) * 1024)
        for name, vs in per.items():
            k = _prefill_name(name)
            if k in ("gram_kernel", "encode_kernel", "bases_kernel", "place_kernel", "count_kernel"):
                res.setdefault(k, {})[counter] = {"kib_mean": float(np.mean(vs)), "dispatches": len(vs),
                                                   "bytes_per_launch": float(np.mean(vs)) * 1024 * scale,
                                                   "scale": scale}
    bj = _json_line(bench_json) if bench_json else None
    alg = {"gram_kernel": bj["breakdown"]["algorithmic_bytes"]["gram_per_layer"],
           "encode_kernel": bj["breakdown"]["algorithmic_bytes"]["encode_per_layer"]} if bj else {}
    rec = {"workload": cfg.name + "-prefill", "prefill_source_sha256": prefill_source_sha(), "kernels": {}}
    lines = [f"# Prefill kernels' HBM traffic, {cfg.name} prompt ({cfg.n_tokens} tokens, {cfg.num_layers} layers)", "",
             "Commands (run from /tmp with TMPDIR=/tmp on one MI355X), then the summary on any host:", "", "```",
             f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch> -o run -- python3 <repo>/bench.py "
             f"--config {ci} {PREFILL_RUN_ARGS}",
             f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write> -o run -- python3 <repo>/bench.py "
             f"--config {ci} {PREFILL_RUN_ARGS}",
             f"python3 <repo>/bench.py --config {ci} --mode prefill --pmc-summary <fetch> <write> "
             f"--bench-json <fetch run's stdout file>", "```", "",
             "Each counter is scaled by (512 MiB) / (its reading for a plain 512 MiB device copy in the same process).",
             "", "| kernel | dispatches | FETCH bytes / launch | WRITE bytes / launch | algorithmic bytes | ratio |",
             "|---|---|---|---|---|---|"]
    for k, v in sorted(res.items()):
        f = v.get("FETCH_SIZE", {}).get("bytes_per_launch", 0.0)
        wr = v.get("WRITE_SIZE", {}).get("bytes_per_launch", 0.0)
        a = alg.get(k)
        rec["kernels"][k] = {"fetch_bytes": f, "write_bytes": wr, "hbm_bytes_per_launch": f + wr,
                             "algorithmic_bytes_per_launch": a, "counters": v}
        lines.append(f"| {k} | {v.get('FETCH_SIZE', {}).get('dispatches', 0)} | {f:.0f} | {wr:.0f} | "
                     f"{'' if a is None else f'{a:.0f}'} | {'' if a is None else f'{(f + wr) / a:.3f}'} |")
    lines += ["", f"Prefill source sha256: `{rec['prefill_source_sha256']}` (bench.py reports `traffic` only while "
                  "the prefill sources and build flags match it)."]
    os.makedirs(PROFILES, exist_ok=True)
    json.dump(rec, open(os.path.join(PROFILES, f"prefill_{cfg.name}_traffic.json"), "w"), indent=1)
    open(os.path.join(PROFILES, f"prefill_{cfg.name}_traffic.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def prefill_stored_traffic(cfg, kernel: str):
    path = os.path.join(PROFILES, f"prefill_{cfg.name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("prefill_source_sha256") != prefill_source_sha():
        return None
    return rec["kernels"].get(kernel, {}).get("hbm_bytes_per_launch")


def prefill_trace_summary(cfg, ci: int, trace_dir: str, bench_json: Optional[str]):
    """profiles/prefill_<workload>_kernel_trace.md from a rocprofv3
    --kernel-trace --stats run of the prefill mode."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = [r for f in files for r in csv.DictReader(open(f)) if _prefill_name(r["Name"])]
    bj = _json_line(bench_json) if bench_json else None
    lines = [f"# Prefill compression kernels, {cfg.name} prompt (batch {cfg.batch}, {cfg.n_tokens} tokens, "
             f"{cfg.num_layers} layers, {cfg.num_kv_heads} KV heads, d {cfg.head_dim}, r_max {cfg.r_max})", "",
             "Command (run from /tmp with TMPDIR=/tmp on one MI355X), then the summary on any host:", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- python3 <repo>/bench.py "
             f"--config {ci} {PREFILL_TRACE_ARGS}",
             f"python3 <repo>/bench.py --config {ci} --mode prefill --trace-summary <out> [--bench-json <default run's stdout file>]",
             "```", "",
             "Per prompt: one Gram launch (+ reduction) and one encode family (count, place, encode, publish; the fp16",
             "basis block copy once per window) per layer, and one bases launch (+ a transpose) per window on a second",
             "stream.  The trace also holds the breakdown's replays: the bases of all windows in one launch (128",
             "workgroups), so the bases row averages launches of 16 and of 128 workgroups.", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {_prefill_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    if bj:
        b, rf = bj["breakdown"], bj["roofline"]
        lines += ["", f"The same build's default `bench.py --config {ci} --mode prefill` run: {bj['value']:.0f} prompt "
                      f"tokens/s ({bj['ms_per_step']:.2f} ms per prompt of {cfg.n_tokens} tokens, {cfg.num_layers} "
                      f"layers); Gram {b['gram_ms']:.2f} ms ({b['gram_GBps']:.0f} GB/s), bases {b['bases_ms']:.2f} ms, "
                      f"encode {b['encode_ms']:.2f} ms ({b['encode_GBps']:.0f} GB/s); dominant kernel "
                      f"{rf['kernel']}: {rf['achieved']:.2f} {rf['unit']} ({rf['frac'] * 100:.1f}% of {rf['peak']})."]
    open(os.path.join(PROFILES, f"prefill_{cfg.name}_kernel_trace.md"), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


def prefill_step_bytes(cfg, tiers) -> dict:
    """Algorithmic bytes of one prefill compression of the whole model, per
    kernel family: the Gram pass reads every prefill key and value once;
    the bases read each window's Gram matrices once and write the bases;
    the encoder reads every key and value and its tier once and writes each
    token at its tier's size plus its position-map entry.  tiers: the
    per-layer tier arrays of one window (they stand for every window)."""
    L, B, H, d, n, lpg = cfg.num_layers, cfg.batch, cfg.num_kv_heads, cfg.head_dim, cfg.n_tokens, cfg.layers_per_group
    kv = B * H * n * d * 2 * 2
    per_tok = np.array([w.compressed_bytes_per_token(r, s, cfg.resid_bits, cfg.coef_bits)
                        for r, s in zip(cfg.tier_rank, cfg.resid_per_tier)])
    enc = []
    for l in range(L):
        t = tiers[l % lpg]
        enc.append(kv + B * H * n + float(per_tok[t.reshape(-1).astype(np.int64)].sum()) + B * H * n * 4)
    bases = cfg.num_groups * (2 * H * d * d * 8 + 2 * H * cfg.r_max * d * 2 * 3)
    return {"gram_per_layer": kv, "encode_per_layer": float(np.mean(enc)), "bases_total": bases,
            "total": kv * L + sum(enc) + bases}


def _gen_prefill_job(args):
    ci, layer, batch, n = args
    from workload.gen import gen_prefill
    return gen_prefill(w.get_config(ci).with_(batch=batch, n_tokens=n), layer)


def run_prefill(args, cfg, K: int, W: int):
    """Prefill compression of the workload's prompt for every layer: Gram
    sums of every layer, the bases of every window in one launch, then the
    bulk encode of every layer.  One window's prefill keys, values and tiers
    (seeded, the generator's distributions) stand in for every window's."""
    import torch
    from workload.gen import gen_sketch, gen_tiers
    from compressed_kv_cache_dwkv_amd import dwkv_reset
    from compressed_kv_cache_dwkv_amd.cache import CompressedKVCache
    L, B, H, d, n, lpg = cfg.num_layers, cfg.batch, cfg.num_kv_heads, cfg.head_dim, cfg.n_tokens, cfg.layers_per_group
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=min(lpg, len(os.sched_getaffinity(0)))) as ex:
        kvs = list(ex.map(_gen_prefill_job, [(args.config, l, cfg.batch, cfg.n_tokens) for l in range(lpg)]))
    tiers = [gen_tiers(cfg, l, n) for l in range(lpg)]
    sketch = min(cfg.r_max + 8, cfg.head_dim)
    omega = gen_sketch(cfg, sketch)
    print(f"bench: prefill inputs generated ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
    torch.cuda.set_device(0)
    cap = [int(c) + 16 for c in max_tier_counts(cfg)]
    cache = CompressedKVCache(L, lpg, cfg.num_q_heads, H, d, cfg.r_max, cfg.tier_rank, cfg.resid_per_tier,
                              cfg.resid_bits, B, cap, n + 16, coef_bits=cfg.coef_bits)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    k_dev = [dev(kv[0]) for kv in kvs]
    v_dev = [dev(kv[1]) for kv in kvs]
    del kvs
    t_dev = [dev(t) for t in tiers]
    om_dev = dev(omega)
    n_dev = torch.full((B,), n, dtype=torch.int32, device="cuda")
    cache.prefill_workspace()
    h = cache.handle
    q = args.power_iters

    def grams():
        for l in range(L):
            cache.prefill_gram(l, k_dev[l % lpg], v_dev[l % lpg], n_dev, first=(l % lpg == 0))

    def bases():
        cache.prefill_bases(0, om_dev, q)

    def encodes():
        dwkv_reset(h)
        for l in range(L):
            cache.prefill_encode(l, k_dev[l % lpg], v_dev[l % lpg], n_dev, t_dev[l % lpg])

    # The step as a pipeline: each window's bases start on a second stream
    # (default priority) as soon as its Gram sums are complete, while the
    # remaining Gram sums run; the encodes of a window wait for its bases
    # only.  The bases read only their window's Gram sums, so they share the
    # workspace with the other calls.
    G = L // lpg
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev_gram = [torch.cuda.Event() for _ in range(G)]
    ev_bases = [torch.cuda.Event() for _ in range(G)]

    def step(s):
        dwkv_reset(h)
        for m in range(G):
            for l in range(m * lpg, (m + 1) * lpg):
                cache.prefill_gram(l, k_dev[l % lpg], v_dev[l % lpg], n_dev, first=(l % lpg == 0))
            ev_gram[m].record(main)
            with torch.cuda.stream(side):
                side.wait_event(ev_gram[m])
                cache.prefill_bases(m, om_dev[m:m + 1], q)
                ev_bases[m].record(side)
        for m in range(G):
            main.wait_event(ev_bases[m])
            for l in range(m * lpg, (m + 1) * lpg):
                cache.prefill_encode(l, k_dev[l % lpg], v_dev[l % lpg], n_dev, t_dev[l % lpg])

    elapsed_ms = _time_graph_steps(step, W, K, 1)
    assert cache.check_errors() == 0, "prefill overflowed the cache"
    gram_ms = _graph_launch_ms(grams, args.kernel_reps)
    bases_ms = _graph_launch_ms(bases, args.kernel_reps)
    enc_ms = _graph_launch_ms(encodes, args.kernel_reps)
    assert cache.check_errors() == 0
    by = prefill_step_bytes(cfg, tiers)
    ms_per_step = elapsed_ms / K
    gram_launch_ms = gram_ms / L
    enc_layer_ms = enc_ms / L
    fam = {"gram": gram_ms, "bases": bases_ms, "encode": enc_ms}
    dominant = max(fam, key=fam.get)
    # the encoder's arithmetic: per vector r d fp32 FMAs for the projection
    # and r d for the residual (2 flops each), K and V of every token
    r_tok = np.asarray(cfg.tier_rank)[np.concatenate([t.reshape(-1) for t in tiers]).astype(np.int64)]
    enc_flop_layer = float(r_tok.sum()) / lpg * d * 2 * 2 * 2
    if dominant == "gram":
        roof = {"bound": "hbm", "kernel": "gram_kernel", "achieved": by["gram_per_layer"] / (gram_launch_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "algorithmic_bytes_per_launch": by["gram_per_layer"],
                "mean_launch_us": gram_launch_ms * 1e3}
    else:
        roof = {"bound": "alu", "kernel": "encode_kernel (+ slot and publish passes)",
                "achieved": enc_flop_layer / (enc_layer_ms * 1e-3) / 1e12, "peak": 157.3, "unit": "TFLOP/s",
                # 157.3 counts two fp32 FMAs per lane and cycle (packed); one per
                # lane and cycle: 256 CUs x 64 lanes x 2 flops x 2.4 GHz
                "peak_unpacked": 78.6,
                "algorithmic_flop_per_launch": enc_flop_layer, "mean_launch_us": enc_layer_ms * 1e3,
                "hbm_GBps": by["encode_per_layer"] / (enc_layer_ms * 1e-3) / 1e9}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if "peak_unpacked" in roof:
        roof["frac_unpacked"] = roof["achieved"] / roof["peak_unpacked"]
    kname = "gram_kernel" if dominant == "gram" else "encode_kernel"
    roof["traffic"] = prefill_stored_traffic(cfg, kname)
    if roof["traffic"] is not None:
        roof["traffic_GBps"] = roof["traffic"] / (roof["mean_launch_us"] * 1e-6) / 1e9
    roof["launch_time_from"] = "replays of a graph of one step's launches of that kernel family"
    res = {
        "metric": PREFILL_METRIC, "value": B * n * K / (elapsed_ms / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp16 inputs; fp16 MFMA + fp32 (Gram), fp64 (bases), fp32 (encoder)",
        "data": "synthetic",
        "config": {"workload": cfg.name + "-prefill", "batch": B, "context": n, "layers": L, "kv_heads": H,
                   "head_dim": d, "layers_per_basis": lpg, "r_max": cfg.r_max, "sketch": sketch,
                   "power_iters": q, "tier_rank": list(cfg.tier_rank), "tier_mix": list(cfg.tier_prob),
                   "resid_channels": cfg.resid_channels, "resid_bits": cfg.resid_bits, "coef_bits": cfg.coef_bits,
                   "inputs": "one window's prefill K/V and tiers stand in for every window's"},
        "step_GBps": by["total"] / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": by["total"] / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "breakdown": {"gram_ms": gram_ms, "bases_ms": bases_ms, "encode_ms": enc_ms, "reset_in_encode": True,
                      "gram_GBps": by["gram_per_layer"] / (gram_launch_ms * 1e-3) / 1e9,
                      "encode_GBps": by["encode_per_layer"] / (enc_layer_ms * 1e-3) / 1e9,
                      "algorithmic_bytes": by},
        "roofline": roof,
        "cpu_baseline": None if args.no_cpu_baseline else prefill_cpu_baseline(cfg, args.cpu_seconds),
    }
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cache.close()
    return res


def prefill_cpu_baseline(cfg, budget_s: float):
    """The oracle's prefill compression on a bounded sample: one window's
    Gram sums and bases over the first n_s tokens, and the bulk encode of
    those tokens for every layer of the window, n_s doubled until the
    budget is spent; scaled to prompt tokens per second over all layers."""
    import oracle
    from workload.gen import gen_prefill, gen_sketch, gen_tiers
    lpg = cfg.layers_per_group
    sketch = min(cfg.r_max + 8, cfg.head_dim)
    omega = gen_sketch(cfg, sketch)[0]
    host = len(os.sched_getaffinity(0))
    threads = min(oracle.max_threads(), host)
    ns, best = 256, None
    total = 0.0
    while total < budget_s and ns <= cfg.n_tokens:
        Ks, Vs, ts = [], [], []
        for l in range(lpg):
            K, V = gen_prefill(cfg, l, n=ns)
            Ks.append(K)
            Vs.append(V)
            ts.append(gen_tiers(cfg, l, ns))
        t0 = time.perf_counter()
        bs = oracle.prefill_bases(cfg, Ks, Vs, [ns] * cfg.batch, omega, 2)
        for l in range(lpg):
            oracle.prefill_encode(cfg, bs["K"], bs["V"], Ks[l], Vs[l], [ns] * cfg.batch, ts[l], nthreads=threads)
        dt = time.perf_counter() - t0
        total += dt
        best = (ns, dt)
        ns *= 2
    ns, dt = best
    return {"value": cfg.batch * ns / (dt * cfg.num_layers / lpg), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "host_cores": host, "cpu_model": _cpu_model(),
            "sample": f"one window ({lpg} layers) of a {ns}-token prompt: Gram sums and bases (fp64 NumPy), "
                      f"then the bulk encode of every token (C, {threads} threads), {dt:.2f} s, "
                      f"scaled to {cfg.num_layers} layers"}


def resolve_config(args):
    """The workload of `--config` with `--coef-bits`, and any `--batch` or
    `--context` override; an overridden workload carries the override in its
    name, so profiles recorded for the workload itself never apply to it."""
    cfg = w.get_config(args.config).with_(coef_bits=args.coef_bits)
    if args.batch and args.batch != cfg.batch:
        cfg = cfg.with_(batch=args.batch, name=f"{cfg.name}-batch{args.batch}")
    if args.context and args.context != cfg.n_tokens:
        cfg = cfg.with_(n_tokens=args.context, name=f"{cfg.name}-ctx{args.context}")
    return cfg


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)
    cfg = resolve_config(args)
    if args.pmc_summary:
        if args.mode == "prefill":
            prefill_pmc_summary(cfg, args.config, *args.pmc_summary, bench_json=args.bench_json)
        else:
            pmc_summary(workload_name(cfg), *args.pmc_summary, bench_json=args.bench_json)
        return
    if args.trace_summary:
        if args.mode == "prefill":
            prefill_trace_summary(cfg, args.config, args.trace_summary, args.bench_json)
        else:
            trace_summary(cfg, args.config, args.trace_summary, args.bench_json)
        return
    K = args.steps if args.steps is not None else cfg.bench_steps
    W = args.warmup
    L, B, H = cfg.num_layers, cfg.batch, cfg.num_kv_heads
    if args.stream_probe:
        print(json.dumps(run_stream_probe(args, cfg, K, W)), flush=True)
        return
    if args.comparator == "dense":
        print(json.dumps(run_dense(args, cfg, K, W)), flush=True)
        return
    if args.mode == "prefill":
        K = args.steps if args.steps is not None else 10
        W = min(W, 2)
        print(json.dumps(run_prefill(args, cfg, K, W)), flush=True)
        return

    # ---- synthetic inputs (host): the layer generators start before the
    #      GPU is touched; each layer is imported as it arrives and dropped
    t0 = time.perf_counter()
    workers = min(16, len(os.sched_getaffinity(0)))
    ex = ProcessPoolExecutor(max_workers=workers)
    layer_iter = ex.map(_gen_layer_job, [(args.config, l, cfg.coef_bits, cfg.batch, cfg.n_tokens) for l in range(L)])
    bases = make_bases(cfg)
    appends = [[gen_append_inputs(cfg, l, s, bases) for l in range(L)] for s in range(W + K)]
    queries = np.stack([gen_query(cfg, l) for l in range(L)])

    import torch
    from compressed_kv_cache_dwkv_amd import dwkv_append, dwkv_decode_attn, dwkv_decode_step
    from compressed_kv_cache_dwkv_amd.cache import CompressedKVCache

    torch.cuda.set_device(0)
    extra = W + K + args.kernel_reps + 8        # appended tokens: steps and kernel timing
    cap = [int(c) + extra for c in max_tier_counts(cfg)]
    cache = CompressedKVCache(L, cfg.layers_per_group, cfg.num_q_heads, H, cfg.head_dim, cfg.r_max,
                              cfg.tier_rank, cfg.resid_per_tier, cfg.resid_bits, B, cap,
                              cfg.n_tokens + extra, decode_splits=args.splits, coef_bits=cfg.coef_bits)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    for m in range(cfg.num_groups):
        cache.set_basis(m, dev(bases["K"][m]), dev(bases["V"][m]))
    for l, lay in enumerate(layer_iter):
        cache.import_layer(l, {k: dev(v) for k, v in lay.items() if k != "n_tokens"},
                           [int(x) for x in lay["n_tokens"]])
        del lay
        if (l + 1) % 8 == 0 or l + 1 == L:
            torch.cuda.synchronize()
            print(f"bench: layer {l + 1}/{L} generated and imported ({time.perf_counter() - t0:.1f} s)",
                  file=sys.stderr, flush=True)
    ex.shutdown()
    torch.cuda.synchronize()
    assert cache.check_errors() == 0, "cache import overflowed"
    q_dev = dev(queries)                                                 # [L][B][Hq][d]
    out_dev = torch.empty((L, B, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    k_dev = dev(np.stack([[appends[s][l]["k"] for l in range(L)] for s in range(W + K)]))
    v_dev = dev(np.stack([[appends[s][l]["v"] for l in range(L)] for s in range(W + K)]))
    t_dev = dev(np.stack([[appends[s][l]["tier"] for l in range(L)] for s in range(W + K)]))
    ws = cache.workspace(B)
    h = cache.handle
    scale = 1.0 / math.sqrt(cfg.head_dim)
    print(f"bench: cache resident ({cache.arena.numel() / 1e9:.2f} GB arena)", file=sys.stderr, flush=True)

    unfused = args.comparator == "unfused"
    if unfused:
        from compressed_kv_cache_dwkv_amd import (dwkv_dense_decode, dwkv_dense_workspace_bytes,
                                                 dwkv_materialize_layer)
        n_cap = (int(cache.cfg.max_tokens) + 63) // 64 * 64
        Kd = torch.empty((B, H, n_cap, cfg.head_dim), dtype=torch.float16, device="cuda")
        Vd = torch.empty((B, H, n_cap // 16, cfg.head_dim, 16), dtype=torch.float16, device="cuda")
        n_dev = torch.empty((B, H), dtype=torch.int32, device="cuda")
        S_dense = _dense_splits(args, cfg)
        ws_dense = torch.zeros(dwkv_dense_workspace_bytes(B, cfg.num_q_heads, H, cfg.head_dim, S_dense),
                               dtype=torch.uint8, device="cuda")

    def layer_step(l, s):
        if unfused:
            dwkv_materialize_layer(h, l, Kd, Vd, n_dev)
            dwkv_dense_decode(q_dev[l], Kd, Vd, n_dev, out_dev[l], ws_dense, S_dense, scale)
            dwkv_append(h, l, k_dev[s, l], v_dev[s, l], t_dev[s, l])
        elif args.separate:
            dwkv_decode_attn(h, l, q_dev[l], out_dev[l], ws, scale)
            dwkv_append(h, l, k_dev[s, l], v_dev[s, l], t_dev[s, l])
        else:
            dwkv_decode_step(h, l, q_dev[l], out_dev[l], ws, k_dev[s, l], v_dev[s, l], t_dev[s, l],
                             softmax_scale=scale)

    def step(s):
        for l in range(L):
            layer_step(l, s)

    for s in range(W):
        step(s)
    torch.cuda.synchronize()

    graphs = []
    if not args.no_graph:
        for c0 in range(W, W + K, args.chunk):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(c0, min(c0 + args.chunk, W + K)):
                    step(s)
            graphs.append(g)
        torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if graphs:
        for g in graphs:
            g.replay()
    else:
        for s in range(W, W + K):
            step(s)
    end.record()
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(end)
    errs = cache.check_errors()
    assert errs == 0, f"device error word {errs}"
    ms_per_step = elapsed_ms / K
    tok_s = B * K / (elapsed_ms / 1e3)

    # ---- decode-kernel duration: every layer's launch of the step (with
    #      its append unless --separate) back to back in one graph, replayed;
    #      events on the launch stream around the replays
    # (counts after the timed steps; the timed launches saw up to K fewer
    # tokens per (layer, KV head): under 0.4% at 64K)
    counts = np.stack([cache.read_counts(l, B) for l in range(L)])     # [L][B][H][T]
    last = appends[W + K - 1]
    layer_bytes = [algorithmic_layer_bytes(cfg, counts[l], None if args.separate else last[l]["tier"])
                   for l in range(L)]
    step_bytes = sum(algorithmic_layer_bytes(cfg, counts[l], last[l]["tier"]) for l in range(L))
    breakdown = None
    if unfused:
        mat_ms = _graph_launch_ms(lambda: [dwkv_materialize_layer(h, l, Kd, Vd, n_dev) for l in range(L)],
                                  args.kernel_reps) / L
        dec_ms = _graph_launch_ms(lambda: [dwkv_dense_decode(q_dev[l], Kd, Vd, n_dev, out_dev[l], ws_dense, S_dense,
                                                             scale) for l in range(L)], args.kernel_reps) / L
        app_ms = _graph_launch_ms(lambda: [dwkv_append(h, l, k_dev[W + K - 1, l], v_dev[W + K - 1, l],
                                                       t_dev[W + K - 1, l]) for l in range(L)], 2) / L
        breakdown = {"materialize_us": mat_ms * 1e3, "dense_decode_us": dec_ms * 1e3, "append_us": app_ms * 1e3,
                     "dense_splits": S_dense, "note": "per layer, from replays of a graph of one step's launches "
                                                      "of each kernel (appends add tokens to the cache)"}
    kg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(kg):
        for l in range(L):
            if unfused:
                dwkv_dense_decode(q_dev[l], Kd, Vd, n_dev, out_dev[l], ws_dense, S_dense, scale)
            elif args.separate:
                dwkv_decode_attn(h, l, q_dev[l], out_dev[l], ws, scale)
            else:
                layer_step(l, W + K - 1)
    kg.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.kernel_reps)]
    torch.cuda._sleep(int(3e8))
    for a, b in ev:
        a.record()
        kg.replay()
        b.record()
    torch.cuda.synchronize()
    assert cache.check_errors() == 0, "kernel timing overflowed the cache"
    durs = np.array([a.elapsed_time(b) for a, b in ev]) / L                              # ms per launch
    graph_launch_ms = float(durs.mean())
    # In the one-launch step every launch of the timed region is the decode
    # kernel, so its average duration is the timed region's time per launch
    # (the replays above, of one step's L launches, also carry each graph
    # launch's own overhead); the two-launch form takes the replays' figure.
    if graphs and not args.separate:
        mean_launch_ms = elapsed_ms / (K * L)
        launch_source = "timed region"
    else:
        mean_launch_ms = graph_launch_ms
        launch_source = "replays of one step's decode launches"
    bytes_per_launch = float(np.mean(layer_bytes))
    kernel_name = "decode_kernel"
    traffic = stored_traffic(workload_name(cfg))
    if unfused:
        # the dense decode over the materialised layer: its dense bytes
        mean_launch_ms = breakdown["dense_decode_us"] * 1e-3
        launch_source = "replays of one step's dense decode launches"
        bytes_per_launch = float(B * H * (cfg.n_tokens + W + K) * cfg.head_dim * 2 * 2)
        kernel_name = "dense_decode_kernel"
        traffic = None
    achieved = bytes_per_launch / (mean_launch_ms * 1e-3) / 1e9

    dense = w.dense_kv_bytes(L, H, cfg.head_dim, cfg.n_tokens + W + K, batch=B)
    res = {
        "metric": METRIC + (" [comparator: unfused decode]" if unfused else ""),
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA operands, fp32 accumulate",
        "data": "synthetic",
        "config": {
            "workload": workload_name(cfg), "batch": B, "context": cfg.n_tokens, "layers": L,
            "q_heads": cfg.num_q_heads, "kv_heads": H, "head_dim": cfg.head_dim,
            "layers_per_basis": cfg.layers_per_group, "r_max": cfg.r_max,
            "tier_rank": list(cfg.tier_rank), "tier_mix": list(cfg.tier_prob),
            "resid_channels": cfg.resid_channels, "resid_bits": cfg.resid_bits,
            "storage": ("fp16 coefficients" if cfg.coef_bits == 16 else
                        "8-bit blockwise coefficients (int8 codes, fp16 block scale per token)")
                       + ", uint8 channel indices, packed codes, fp16 scales",
            "coef_bits": cfg.coef_bits,
            "graph_replay": bool(graphs), "decode_splits": cache.splits,
            "launches_per_layer": 3 if unfused else 2 if args.separate else 1,
            **({"comparator": "unfused"} if unfused else {}),
        },
        "step_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
            "traffic_GBps": None if traffic is None else traffic / (mean_launch_ms * 1e-3) / 1e9,
            "kernel": kernel_name, "algorithmic_bytes_per_launch": bytes_per_launch,
            "mean_launch_us": mean_launch_ms * 1e3, "launch_time_from": launch_source,
            "one_step_graph_launch_us": graph_launch_ms * 1e3,
        },
        **({"breakdown": breakdown} if breakdown else {}),
        "memory": {
            "compressed_bytes": step_bytes, "dense_fp16_bytes": dense,
            "reduction_vs_fp16": dense / step_bytes,
        },
        "paper_context": {"decode_tok_s_64k": 72.8, "kv_memory_reduction": 8.3,
                          "note": "end-to-end generation on unstated hardware and model; not comparable"},
    }
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, bases, appends, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    cache.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
