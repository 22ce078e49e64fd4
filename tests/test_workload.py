"""Generator and byte-accounting pins (CPU)."""
import json
import os

import numpy as np
import pytest

import workload as w
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases
from tests.helpers import tiny_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_dense_kv_size_matches_printed_example():
    ex = json.load(open(os.path.join(GOLDEN, "kv_size_example.json")))
    n = w.dense_kv_bytes(ex["layers"], ex["kv_heads"], ex["head_dim"], ex["tokens"],
                         elem_bytes=ex["bytes_per_element"])
    assert n == 32_768_000_000
    assert round(n / 1e9, 1) == ex["printed_total_gb"]


def test_compressed_bytes_per_token():
    # rank 8, s = 8 INT4: 2*8*2 (K,V coef) + 2*(8 + 4 + 2) (K,V residual blocks)
    assert w.compressed_bytes_per_token(8, 8, 4) == 32 + 28
    assert w.compressed_bytes_per_token(64, 8, 4) == 256 + 28
    assert w.compressed_bytes_per_token(4, 4, 8) == 16 + 2 * (4 + 4 + 2)
    assert w.compressed_bytes_per_token(16, 0, 4) == 64
    c = w.get_config(2)
    mean = sum(p * w.compressed_bytes_per_token(r, 8, 4) for r, p in zip(c.tier_rank, c.tier_prob))
    assert abs(mean - 97.44) < 1e-9


def test_determinism_and_independence_of_fields():
    cfg = tiny_config(n_tokens=64)
    a = gen_layer(cfg, 1)
    b = gen_layer(cfg, 1)
    for k in a:
        assert np.array_equal(a[k], b[k])
    c = gen_layer(cfg, 0)
    assert not np.array_equal(a["coefK"], c["coefK"])
    # tiers are shared by the layers of one depth group
    assert np.array_equal(a["tier"], c["tier"])
    q0, q1 = gen_query(cfg, 0, 0), gen_query(cfg, 0, 1)
    assert not np.array_equal(q0, q1)


def test_tier_mix_and_value_ranges():
    cfg = w.get_config(1)
    lay = gen_layer(cfg, 0, n=16384)
    t = lay["tier"].ravel()
    N = t.size
    for k, p in enumerate(cfg.tier_prob):
        f = np.mean(t == k)
        assert abs(f - p) <= 5 * np.sqrt(p * (1 - p) / N)
    for z in "KV":
        coef = lay["coef" + z].astype(np.float64)
        r = np.asarray(cfg.tier_rank)[lay["tier"]]
        mask = np.arange(cfg.r_max)[None, None, None, :] >= r[..., None]
        assert not coef[mask].any()
        # variance of c_i is 1/(1+i)
        for i in (0, 3, 7):
            v = coef[..., i].ravel()
            assert abs(v.var() / (1.0 / (1 + i)) - 1) < 0.05
        idx = lay["idx" + z].astype(int)
        assert (np.diff(idx, axis=-1) > 0).all() and idx.max() < cfg.head_dim
        val = lay["val" + z]
        assert val.min() >= -7 and val.max() <= 7 and len(np.unique(val)) == 15
        sc = lay["scale" + z].astype(np.float64)
        assert (sc >= 0).all() and abs(sc.mean() - 0.01 * np.sqrt(2 / np.pi)) < 2e-4


def test_router_skew_forces_top_tier():
    cfg = w.get_config(3).with_(batch=2)
    lay = gen_layer(cfg, 0, n=4096)
    top = cfg.num_tiers - 1
    assert (lay["tier"][:, :, :64] == top).all()
    forced = (lay["tier"] == top).all(axis=1)   # forced positions are top for every head
    assert forced.sum(axis=1).min() >= 64 + round(0.02 * 4096) - 5


def test_bases_are_orthonormal_in_fp16():
    for i in (0, 1):
        cfg = w.get_config(i)
        b = make_bases(cfg)
        for z in "KV":
            B = b[z][0, 0].astype(np.float64)
            assert np.abs(B @ B.T - np.eye(cfg.r_max)).max() <= 2e-3
            B64 = b[z + "64"][0, 0]
            assert np.abs(B64.T @ B64 - np.eye(cfg.r_max)).max() <= 1e-12


def test_append_inputs_shapes():
    cfg = w.get_config(0)
    b = make_bases(cfg)
    a = gen_append_inputs(cfg, 1, 3, b)
    assert a["k"].shape == (1, 1, 64) and a["k"].dtype == np.float16
    assert a["tier"].max() < cfg.num_tiers
