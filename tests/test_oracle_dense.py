"""Pins of oracle.materialize and oracle.dense_decode (CPU).

materialize is Eq. (1) of the paper (§3 Method) for every cached token;
dense_decode is textbook softmax attention over a dense fp16 cache.  Both
are checked against independent routes: NumPy's einsum materialisation,
torch's scaled_dot_product_attention in fp64 (a library routine), exact
identity bases and closed forms."""
import numpy as np
import pytest

import oracle
from workload.gen import gen_layer, gen_query, make_bases
from tests.helpers import dense_from_logical, sdpa_fp64, tiny_config


def _cfg(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=32, r_max=16, tier_rank=(4, 8, 16),
                tier_prob=(0.5, 0.3, 0.2), resid_channels=3, resid_bits=4, n_tokens=40)
    base.update(kw)
    return tiny_config(**base)


def test_materialize_matches_numpy_einsum():
    cfg = _cfg()
    bases = make_bases(cfg)
    lay = gen_layer(cfg, 1)
    lay["n_tokens"][:] = [40, 23]
    K, V = oracle.materialize(cfg, lay, bases["K"][0], bases["V"][0])
    for z, got in (("K", K), ("V", V)):
        ref = dense_from_logical(cfg, lay, bases[z][0], z)
        assert np.abs(got[0] - ref[0]).max() <= 1e-12
        assert np.abs(got[1, :, :23] - ref[1, :, :23]).max() <= 1e-12
        assert not got[1, :, 23:].any()


def test_materialize_identity_basis_is_exact():
    """B = I, r = d for the top tier: K^ = c + scale * code on the kept channels, exactly."""
    cfg = _cfg(head_dim=16, r_max=16, tier_rank=(16,), tier_prob=(1.0,), resid_channels=2, resid_bits=8)
    bases = make_bases(cfg, identity=True)
    lay = gen_layer(cfg, 0)
    K, V = oracle.materialize(cfg, lay, bases["K"][0], bases["V"][0])
    ref = lay["coefK"].astype(np.float64).copy()
    sc = lay["scaleK"].astype(np.float64)
    for b in range(cfg.batch):
        for h in range(cfg.num_kv_heads):
            for t in range(cfg.n_tokens):
                for u in range(2):
                    ref[b, h, t, lay["idxK"][b, h, t, u]] += sc[b, h, t] * lay["valK"][b, h, t, u]
    assert np.array_equal(K, ref)


@pytest.mark.parametrize("seed", range(3))
def test_dense_decode_equals_sdpa(seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, n = 3, 8, 2, 64, 50
    K = rng.standard_normal((B, Hkv, n, d)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float16)
    q = (rng.standard_normal((B, Hq, d)) * 2).astype(np.float16)
    ns = [50, 17, 1]
    got = oracle.dense_decode(K, V, ns, q)
    ref = sdpa_fp64(q, K.astype(np.float64), V.astype(np.float64), ns, 1.0 / np.sqrt(d))
    assert np.abs(got - ref).max() <= 1e-12


def test_dense_decode_closed_forms():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, d, n = 1, 4, 1, 16, 30
    K = rng.standard_normal((B, Hkv, n, d)).astype(np.float16)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float16)
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    # one token: its value
    one = oracle.dense_decode(K, V, [1], q)
    assert np.abs(one[0] - V[0, 0, 0].astype(np.float64)[None, :]).max() <= 1e-15
    # zero query: the mean value
    z = oracle.dense_decode(K, V, [n], np.zeros_like(q))
    assert np.abs(z[0] - V[0, 0].astype(np.float64).mean(0)[None, :]).max() <= 1e-14
    # empty context: zeros
    assert not oracle.dense_decode(K, V, [0], q).any()


def test_dense_decode_of_materialised_cache_matches_compressed_decode():
    """Attention over fp16-rounded K^, V^ equals the compressed oracle up to
    that rounding (2^-11 relative per element)."""
    cfg = _cfg(head_dim=64, r_max=32, tier_rank=(8, 16, 32), n_tokens=200)
    bases = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    q = gen_query(cfg, 0)
    K, V = oracle.materialize(cfg, lay, bases["K"][0], bases["V"][0])
    dense = oracle.dense_decode(K.astype(np.float16), V.astype(np.float16), lay["n_tokens"], q)
    comp = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)
    err = np.abs(dense - comp).max(-1) / np.abs(comp).max(-1)
    assert err.max() <= 2e-3
