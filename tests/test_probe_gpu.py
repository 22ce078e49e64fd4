"""dwkv_probe_error (the paper's Eq. (3) attention-output probe) through the
C ABI against oracle.probe_error (needs an MI355X).

The probe's two attention outputs each meet the decode's 2e-3 row-max
bound, so the GPU error e differs from the oracle's by about that bound
times the row max over the row norm: the test allows 5e-3 absolute plus 2%
of e."""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_layer, gen_query, make_bases
from tests.helpers import tiny_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _block_v(v):
    B, H, n_cap, d = v.shape
    return np.ascontiguousarray(v.reshape(B, H, n_cap // 16, 16, d).transpose(0, 1, 2, 4, 3))


def _probe(G, cfg, lay, bases, K, V, qs, layer, dense_splits=8):
    import torch
    import compressed_kv_cache_dwkv_amd as d
    B, H = cfg.batch, cfg.num_kv_heads
    n_cap = K.shape[2]
    cache = G.make_cache(cfg, n=int(lay["n_tokens"].max()))
    try:
        m = layer // cfg.layers_per_group
        G.load_bases(cache, bases, groups=[m])
        G.load_layer(cache, layer, lay)
        ws = torch.zeros(d.dwkv_probe_workspace_bytes(cache.cfg, B, len(qs), dense_splits), dtype=torch.uint8,
                         device="cuda")
        err = torch.empty((B, H), dtype=torch.float32, device="cuda")
        n_ref = G.dev(np.repeat(lay["n_tokens"].astype(np.int32)[:, None], H, 1))
        q = G.dev(np.stack(qs))
        print(f"probe test: {cfg.name} B={B} n={lay['n_tokens']} queries={len(qs)}", flush=True)
        outs = []
        for _ in range(2):                       # the workspace is ready for the next call
            d.dwkv_probe_error(cache.handle, layer, q, G.dev(K), G.dev(_block_v(V)), n_ref, err, ws, dense_splits)
            torch.cuda.synchronize()
            outs.append(err.cpu().numpy().astype(np.float64))
        assert np.array_equal(outs[0], outs[1])
        assert cache.check_errors() == 0
        return outs[0]
    finally:
        cache.close()


@pytest.mark.parametrize("noise", [0.02, 0.1])
def test_probe_error_matches_oracle(G, noise):
    cfg = w.get_config(1).with_(batch=2)
    n = 3000
    layer = 5
    m = layer // cfg.layers_per_group
    bases = make_bases(cfg)
    lay = gen_layer(cfg, layer, n=n)
    lay["n_tokens"][:] = [3000, 2100]
    Kc, Vc = oracle.materialize(cfg, lay, bases["K"][m], bases["V"][m])
    rng = np.random.default_rng(int(noise * 1000))
    n_cap = 3008
    K = np.zeros((cfg.batch, cfg.num_kv_heads, n_cap, cfg.head_dim), np.float16)
    V = np.zeros_like(K)
    K[:, :, :n] = (Kc + noise * rng.standard_normal(Kc.shape)).astype(np.float16)
    V[:, :, :n] = (Vc + noise * rng.standard_normal(Vc.shape)).astype(np.float16)
    qs = [gen_query(cfg, layer, step=i) for i in range(3)]
    ref = oracle.probe_error(cfg, lay, bases["K"][m], bases["V"][m], K[:, :, :n], V[:, :, :n], lay["n_tokens"], qs)
    got = _probe(G, cfg, lay, bases, K, V, qs, layer)
    assert ref.min() > 0.01
    assert np.all(np.abs(got - ref) <= 5e-3 + 0.02 * ref), (got, ref)


def test_probe_error_near_zero_for_an_exact_cache(G):
    """B = I, r = d, no residual: the compressed cache holds the reference
    exactly, so the error is only the two kernels' rounding."""
    cfg = tiny_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=64, r_max=64, tier_rank=(64,),
                      tier_prob=(1.0,), tier_resid=(0,), resid_channels=0, resid_bits=4, n_tokens=1000)
    bases = make_bases(cfg, identity=True)
    lay = gen_layer(cfg, 0)
    n_cap = 1024
    K = np.zeros((2, 2, n_cap, 64), np.float16)
    V = np.zeros_like(K)
    K[:, :, :1000] = lay["coefK"]
    V[:, :, :1000] = lay["coefV"]
    qs = [gen_query(cfg, 0, step=i) for i in range(2)]
    got = _probe(G, cfg, lay, bases, K, V, qs, 0, dense_splits=3)
    assert got.max() <= 5e-3
