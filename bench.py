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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workload as w  # noqa: E402
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases, max_tier_counts  # noqa: E402

METRIC = "decode tokens/s + achieved HBM GB/s (% of peak), compressed-KV attn at 64K"
PEAK_HBM_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "compressed_kv_cache_dwkv_amd", "csrc", "decode.hip")


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's)")
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--config", type=int, default=2, help="workload index 0-4 (2 = 64K headline)")
    p.add_argument("--chunk", type=int, default=16, help="steps per captured graph")
    p.add_argument("--splits", type=int, default=0, help="decode workgroups per KV head (0 = auto)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="launch eagerly instead of graph replay")
    p.add_argument("--kernel-reps", type=int, default=10)
    p.add_argument("--separate", action="store_true",
                   help="two launches per layer (dwkv_decode_attn, dwkv_append) instead of dwkv_decode_step")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 512 MiB device copy (counter calibration)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                        "script with --copy-probe into profiles/ and exit")
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


def pmc_summary(workload: str, fetch_dir: str, write_dir: str):
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
           "decode_source_sha256": hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest(),
           "hbm_bytes_per_launch": total, "counters": res,
           "copy_probe_bytes": COPY_PROBE_BYTES}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.json")
    json.dump(rec, open(path, "w"), indent=1)
    print(json.dumps(rec), flush=True)


def _gen_layer_job(args):
    ci, layer = args
    return gen_layer(w.get_config(ci), layer)


def algorithmic_layer_bytes(cfg, counts: np.ndarray) -> int:
    """Bytes the method must move for one layer's decode: every cached token at
    its tier's size (fp16 coefficients at the routed rank, residual indices,
    packed codes, scale; K and V), both bases of every KV head (once: every
    sequence shares them), q and out."""
    per_tok = np.array([w.compressed_bytes_per_token(r, s, cfg.resid_bits)
                        for r, s in zip(cfg.tier_rank, cfg.resid_per_tier)])
    tok = float((counts.reshape(-1, cfg.num_tiers) * per_tok[None, :]).sum())
    bases = 2 * cfg.num_kv_heads * cfg.r_max * cfg.head_dim * 2
    qo = cfg.batch * cfg.num_q_heads * cfg.head_dim * (2 + 4)
    return int(tok + bases + qo)


def append_layer_bytes(cfg, tier: np.ndarray) -> int:
    """Bytes one layer's append moves beyond the bases (which the decode in
    the same launch reads): the new K and V and the tier per (b, KV head) in,
    the encoded token, its tier count and its position-map entry out."""
    per_tok = np.array([w.compressed_bytes_per_token(r, s, cfg.resid_bits)
                        for r, s in zip(cfg.tier_rank, cfg.resid_per_tier)])
    ins = tier.size * (2 * cfg.head_dim * 2 + 1)
    outs = float(per_tok[tier.reshape(-1).astype(np.int64)].sum()) + tier.size * 8
    return int(ins + outs)


def stored_traffic(workload: str):
    """HBM bytes per decode launch measured by rocprofv3 counters, if the
    summary in profiles/ was taken on the current decode kernel source."""
    path = os.path.join(PROFILES, f"decode_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    if rec.get("decode_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, bases, appends, budget_s: float):
    """The oracle's decode + append, layer by layer over one step (each
    layer's synthetic input regenerated first, outside the timing), until
    the budget is spent; scaled to a full step."""
    import oracle
    threads = oracle.max_threads()
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
    step_s = dt / done * cfg.num_layers
    used = min(threads, cfg.batch * cfg.num_kv_heads)
    return {
        "value": cfg.batch / step_s, "unit": "tokens/s", "cores": used, "kind": "oracle",
        "sample": f"{done} of {cfg.num_layers} layers of one step (decode over all "
                  f"{cfg.n_tokens} tokens x {cfg.batch * cfg.num_kv_heads} KV heads + append), "
                  f"{dt:.1f} s, scaled to a full step",
    }


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)
    cfg = w.get_config(args.config)
    if args.pmc_summary:
        pmc_summary(cfg.name, *args.pmc_summary)
        return
    K = args.steps if args.steps is not None else cfg.bench_steps
    W = args.warmup
    L, B, H = cfg.num_layers, cfg.batch, cfg.num_kv_heads

    # ---- synthetic inputs (host): the layer generators start before the
    #      GPU is touched; each layer is imported as it arrives and dropped
    t0 = time.perf_counter()
    workers = min(16, len(os.sched_getaffinity(0)))
    ex = ProcessPoolExecutor(max_workers=workers)
    layer_iter = ex.map(_gen_layer_job, [(args.config, l) for l in range(L)])
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
                              cfg.n_tokens + extra, decode_splits=args.splits)
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

    def layer_step(l, s):
        if args.separate:
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
    counts = np.stack([cache.read_counts(l, B) for l in range(L)])     # [L][B][H][T]
    app_bytes = [0 if args.separate else append_layer_bytes(cfg, appends[W + K - 1][l]["tier"])
                 for l in range(L)]
    layer_bytes = [algorithmic_layer_bytes(cfg, counts[l]) + app_bytes[l] for l in range(L)]
    step_bytes = sum(algorithmic_layer_bytes(cfg, counts[l]) +
                     append_layer_bytes(cfg, appends[W + K - 1][l]["tier"]) for l in range(L))
    kg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(kg):
        for l in range(L):
            if args.separate:
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
    achieved = bytes_per_launch / (mean_launch_ms * 1e-3) / 1e9
    traffic = stored_traffic(cfg.name)

    dense = w.dense_kv_bytes(L, H, cfg.head_dim, cfg.n_tokens + W + K, batch=B)
    res = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "batch": B, "context": cfg.n_tokens, "layers": L,
            "q_heads": cfg.num_q_heads, "kv_heads": H, "head_dim": cfg.head_dim,
            "layers_per_basis": cfg.layers_per_group, "r_max": cfg.r_max,
            "tier_rank": list(cfg.tier_rank), "tier_mix": list(cfg.tier_prob),
            "resid_channels": cfg.resid_channels, "resid_bits": cfg.resid_bits,
            "storage": "fp16 coefficients, uint8 channel indices, packed codes, fp16 scales",
            "graph_replay": bool(graphs),
            "launches_per_layer": 2 if args.separate else 1,
        },
        "step_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
            "kernel": "decode_kernel", "algorithmic_bytes_per_launch": bytes_per_launch,
            "mean_launch_us": mean_launch_ms * 1e3, "launch_time_from": launch_source,
            "one_step_graph_launch_us": graph_launch_ms * 1e3,
        },
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
