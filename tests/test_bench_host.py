"""bench.py's host logic (CPU): the byte accounting every roofline figure
divides by, checked against a count token by token from the storage format
(K and V coefficients at the token's routed rank, and per K and V a
residual block of s index bytes, s codes of `bits` bits and one fp16
scale), plus hand values; the refusal of more than one GPU; and that the
source hashes tying recorded counter traffic to a build cover every file
the profiled kernels include."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workload as w
from workload.gen import gen_layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


def _token_bytes(rank, s, bits, coef_bits):
    coef = 2 * rank if coef_bits == 16 else rank + 2        # fp16, or int8 codes + one fp16 block scale
    resid = 0 if s == 0 else s + (s * bits + 7) // 8 + 2    # indices, packed codes, fp16 scale
    return 2 * coef + 2 * resid


# (config 3 at batch 16: the bases count once per KV head, not per sequence)
@pytest.mark.parametrize("ci,coef_bits", [(0, 16), (0, 8), (1, 16), (3, 16)])
def test_layer_bytes_match_a_token_by_token_count(bench, ci, coef_bits):
    cfg = w.get_config(ci).with_(coef_bits=coef_bits)
    if ci in (1, 3):
        cfg = cfg.with_(n_tokens=2048 if ci == 1 else 256)
    lay = gen_layer(cfg, 0)
    tiers, n_tok = np.asarray(lay["tier"]), np.asarray(lay["n_tokens"])
    B, H, T = cfg.batch, cfg.num_kv_heads, cfg.num_tiers
    counts = np.zeros((B, H, T), np.int64)
    brute = 0
    for b in range(B):
        for h in range(H):
            for t in tiers[b, h, :int(n_tok[b])]:
                counts[b, h, t] += 1
                brute += _token_bytes(cfg.tier_rank[t], cfg.resid_per_tier[t], cfg.resid_bits, coef_bits)
    bases = 2 * H * cfg.r_max * cfg.head_dim * 2                  # B_K and B_V, fp16, once per KV head
    app = np.arange(B * H).reshape(B, H) % T                      # one appended token per (sequence, KV head)
    app_bytes = sum(_token_bytes(cfg.tier_rank[t], cfg.resid_per_tier[t], cfg.resid_bits, coef_bits)
                    for t in app.reshape(-1))
    assert bench.algorithmic_layer_bytes(cfg, counts) == brute + bases
    assert bench.algorithmic_layer_bytes(cfg, counts, app) == brute + bases + app_bytes


def test_token_bytes_by_hand():
    # rank 8, 8 residual channels of 4-bit codes: 2 x 16 B coefficients + 2 x (8 + 4 + 2) B
    assert w.compressed_bytes_per_token(8, 8, 4) == 60
    assert w.compressed_bytes_per_token(64, 8, 4) == 284
    # 8-bit coefficients: rank codes plus a 2-byte block scale per K and V
    assert w.compressed_bytes_per_token(8, 8, 4, coef_bits=8) == 2 * 10 + 28
    # no residual channels: no residual block at all
    assert w.compressed_bytes_per_token(16, 0, 4) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _local_includes(path, seen):
    """`path` and every file it reaches through #include "..." (transitively),
    looked up beside the including file, then in include/."""
    import re
    path = os.path.realpath(path)
    if path in seen:
        return seen
    seen.add(path)
    for line in open(path):
        m = re.match(r'\s*#\s*include\s+"([^"]+)"', line)
        if m:
            for d in (os.path.dirname(path), os.path.join(ROOT, "include")):
                cand = os.path.join(d, m.group(1))
                if os.path.exists(cand):
                    _local_includes(cand, seen)
                    break
            else:
                raise AssertionError(f"{path}: include {m.group(1)} not found")
    return seen


@pytest.mark.parametrize("kind,units", [("decode", ("decode.hip", "decode8.hip")), ("prefill", ("prefill.hip",))])
def test_source_hash_covers_every_included_file(bench, kind, units):
    csrc = os.path.join(ROOT, "compressed_kv_cache_dwkv_amd", "csrc")
    reached = set()
    for u in units:
        _local_includes(os.path.join(csrc, u), reached)
    hashed = {os.path.realpath(f) for f in (bench.DECODE_SRCS if kind == "decode" else bench.PREFILL_SRCS)}
    missing = sorted(os.path.relpath(f, ROOT) for f in reached - hashed)
    assert not missing, f"{kind} hash misses {missing}"
    assert os.path.realpath(os.path.join(ROOT, "compressed_kv_cache_dwkv_amd", "build.py")) in hashed


def test_overridden_workloads_take_no_recorded_traffic(bench, monkeypatch):
    def cfg_of(*argv):
        monkeypatch.setattr(sys, "argv", ["bench.py", *argv])
        return bench.resolve_config(bench.parse_args())
    base = cfg_of()
    assert base.name == "llama3-8b-64k" and base.batch == 1 and base.n_tokens == 65536
    assert bench.stored_traffic(bench.workload_name(base)) is not None
    for argv, field, value, name in ((("--context", "8192"), "n_tokens", 8192, "llama3-8b-64k-ctx8192"),
                                     (("--batch", "4"), "batch", 4, "llama3-8b-64k-batch4"),
                                     (("--config", "3", "--batch", "2"), "batch", 2, "llama3-8b-32k-b16-batch2")):
        cfg = cfg_of(*argv)
        assert getattr(cfg, field) == value and cfg.name == name
        assert bench.stored_traffic(bench.workload_name(cfg)) is None
    same = cfg_of("--context", "65536", "--batch", "1")       # the workload's own values: not an override
    assert same.name == base.name
