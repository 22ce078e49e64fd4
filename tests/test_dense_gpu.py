"""The uncompressed comparators through the C ABI against the oracle (needs
an MI355X): dwkv_materialize_layer against oracle.materialize (Eq. (1)),
dwkv_dense_decode against oracle.dense_decode (textbook attention over a
dense fp16 cache), and the unfused decode (materialise, then dense decode)
against oracle.decode over the compressed cache.

Tolerances: the materialised fp16 values are the fp32 sum of exact fp16
products plus the residual, rounded once, so each is within one fp16 unit
in the last place of the exact fp64 value; attention outputs meet the same
2e-3 row-max-normalised bound as the compressed decode."""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_layer, gen_query, make_bases

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _round64(n):
    return (n + 63) // 64 * 64


def _unblock_v(v, n_cap, d):
    """[B][H][n_cap/16][d][16] -> [B][H][n_cap][d]."""
    B, H = v.shape[:2]
    return v.reshape(B, H, n_cap // 16, d, 16).transpose(0, 1, 2, 4, 3).reshape(B, H, n_cap, d)


def _block_v(v):
    """[B][H][n_cap][d] -> [B][H][n_cap/16][d][16]."""
    B, H, n_cap, d = v.shape
    return np.ascontiguousarray(v.reshape(B, H, n_cap // 16, 16, d).transpose(0, 1, 2, 4, 3))


def _materialize(G, cache, layer, batch, cfg, n_cap):
    import torch
    import compressed_kv_cache_dwkv_amd as d
    H, D = cfg.num_kv_heads, cfg.head_dim
    ko = torch.full((batch, H, n_cap, D), float("nan"), dtype=torch.float16, device="cuda")
    vo = torch.full((batch, H, n_cap // 16, D, 16), float("nan"), dtype=torch.float16, device="cuda")
    no = torch.zeros((batch, H), dtype=torch.int32, device="cuda")
    d.dwkv_materialize_layer(cache.handle, layer, ko, vo, no)
    torch.cuda.synchronize()
    return ko, vo, no


@pytest.mark.parametrize("ci,n,ragged,cb", [(0, None, None, 16), (1, 3000, [3000, 1777], 16), (4, 2000, None, 16),
                                           (1, 3000, [3000, 1777], 8), (0, None, None, 8)])
def test_materialize_matches_oracle_within_one_ulp(G, ci, n, ragged, cb):
    cfg = w.get_config(ci).with_(coef_bits=cb)
    if ragged:
        cfg = cfg.with_(batch=len(ragged))
    n = cfg.n_tokens if n is None else n
    bases = make_bases(cfg)
    cache = G.make_cache(cfg, n=n)
    layer = 1
    m = layer // cfg.layers_per_group
    try:
        G.load_bases(cache, bases, groups=[m])
        lay = gen_layer(cfg, layer, n=n)
        if ragged:
            lay["n_tokens"][:] = ragged
        G.load_layer(cache, layer, lay)
        n_cap = _round64(n + 16)
        ko, vo, no = _materialize(G, cache, layer, cfg.batch, cfg, n_cap)
        K, V = oracle.materialize(cfg, lay, bases["K"][m], bases["V"][m])
        gk = ko.cpu().numpy()
        gv = _unblock_v(vo.cpu().numpy(), n_cap, cfg.head_dim)
        assert np.array_equal(no.cpu().numpy(), np.repeat(lay["n_tokens"][:, None], cfg.num_kv_heads, 1))
        for got, ref in ((gk, K), (gv, V)):
            for b in range(cfg.batch):
                nb = int(lay["n_tokens"][b])
                g = got[b, :, :nb].astype(np.float64)
                r = ref[b, :, :nb]
                ulp = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
                assert np.all(np.abs(g - r) <= ulp), f"b={b}: {np.abs(g - r).max()}"
                # the rest of the last 64-token chunk is written as zeros
                tail = got[b, :, nb:_round64(nb)]
                assert not tail.astype(np.float32).any()
    finally:
        cache.close()


@pytest.mark.parametrize("gq,d,ns,splits", [
    (4, 128, [1000, 0, 31, 33], 3),
    (1, 64, [64, 65, 500], 1),
    (2, 128, [2000, 1], 16),
    (8, 128, [3000], 64),
    (8, 64, [257, 12], 5),
])
def test_dense_decode_matches_oracle(G, gq, d, ns, splits):
    import torch
    import compressed_kv_cache_dwkv_amd as dw
    rng = np.random.default_rng(gq * 1000 + d + len(ns))
    B, Hkv = len(ns), 2
    Hq = gq * Hkv
    n_cap = _round64(max(ns) + 1)
    K = rng.standard_normal((B, Hkv, n_cap, d)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, n_cap, d)).astype(np.float16)
    for peak in (1.0, 8.0):
        q = (rng.standard_normal((B, Hq, d)) * peak).astype(np.float16)
        ref = oracle.dense_decode(K, V, ns, q)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        ws = torch.zeros(dw.dwkv_dense_workspace_bytes(B, Hq, Hkv, d, splits), dtype=torch.uint8, device="cuda")
        n_dev = G.dev(np.repeat(np.asarray(ns, np.int32)[:, None], Hkv, 1))
        print(f"dense test: gq={gq} d={d} n={ns} splits={splits} peak={peak}", flush=True)
        for rep in range(2):                       # the workspace is left ready for the next call
            dw.dwkv_dense_decode(G.dev(q), G.dev(K), G.dev(_block_v(V)), n_dev, out, ws, splits)
            torch.cuda.synchronize()
            got = out.cpu().numpy().astype(np.float64)
            for b, n in enumerate(ns):
                if n == 0:
                    assert not got[b].any()
                    continue
                err = G.norm_err(got[b], ref[b])
                assert err.max() <= TOL, f"b={b} n={n}: {err.max():.3e}"


def test_dense_decode_full_size_64k(G):
    """The dense baseline at the 64K Llama-3-8B shape (one layer, 8 KV
    heads, 32 query heads), every head against the oracle."""
    import torch
    import compressed_kv_cache_dwkv_amd as dw
    cfg = w.get_config(2)
    rng = np.random.default_rng(2)
    B, Hkv, Hq, d, n = 1, cfg.num_kv_heads, cfg.num_q_heads, cfg.head_dim, cfg.n_tokens
    K = rng.standard_normal((B, Hkv, n, d)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    ref = oracle.dense_decode(K, V, [n], q)
    splits = 32
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.zeros(dw.dwkv_dense_workspace_bytes(B, Hq, Hkv, d, splits), dtype=torch.uint8, device="cuda")
    dw.dwkv_dense_decode(G.dev(q), G.dev(K), G.dev(_block_v(V)), G.dev(np.full((B, Hkv), n, np.int32)), out, ws,
                         splits)
    torch.cuda.synchronize()
    err = G.norm_err(out.cpu().numpy().astype(np.float64), ref)
    assert err.max() <= TOL, f"{err.max():.3e}"


@pytest.mark.parametrize("ci,n", [(1, None), (2, None)])
def test_unfused_decode_matches_compressed_oracle(G, ci, n):
    """Materialise the layer, then dense attention over it: the decode the
    fused kernel replaces, against the oracle over the compressed cache."""
    import torch
    import compressed_kv_cache_dwkv_amd as dw
    cfg = w.get_config(ci)
    n = cfg.n_tokens if n is None else n
    bases = make_bases(cfg)
    cache = G.make_cache(cfg, n=n)
    layer = 6
    m = layer // cfg.layers_per_group
    try:
        G.load_bases(cache, bases, groups=[m])
        lay = gen_layer(cfg, layer, n=n)
        G.load_layer(cache, layer, lay)
        n_cap = _round64(cache.cfg.max_tokens)
        ko, vo, no = _materialize(G, cache, layer, cfg.batch, cfg, n_cap)
        q = gen_query(cfg, layer)
        splits = 32
        out = torch.empty((cfg.batch, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
        ws = torch.zeros(dw.dwkv_dense_workspace_bytes(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads,
                                                       cfg.head_dim, splits), dtype=torch.uint8, device="cuda")
        dw.dwkv_dense_decode(G.dev(q), ko, vo, no, out, ws, splits)
        torch.cuda.synchronize()
        ref = oracle.decode(cfg, lay, bases["K"][m], bases["V"][m], q)
        err = G.norm_err(out.cpu().numpy().astype(np.float64), ref)
        assert err.max() <= TOL, f"{err.max():.3e}"
        assert cache.check_errors() == 0
    finally:
        cache.close()
