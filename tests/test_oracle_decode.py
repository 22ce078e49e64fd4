"""Pins of oracle.decode (CPU, no GPU): library routine, closed forms, invariants."""
import math

import numpy as np
import pytest

import oracle
from workload import gen as wg
from workload.gen import empty_layer, gen_layer, gen_query, make_bases
from tests.helpers import dense_from_logical, rel_err, sdpa_fp64, signed_permutation_basis, tiny_config


def _alpha(cfg):
    return 1.0 / math.sqrt(cfg.head_dim)


# ------------------------------------------------------------ library routine
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_identity_basis_equals_sdpa(seed):
    """B = I: the cache holds K and V directly (coefficients + sparse residual);
    decode must equal torch's fp64 scaled_dot_product_attention on them."""
    cfg = tiny_config(seed=seed, n_tokens=9)
    bases = make_bases(cfg, identity=True)
    lay = gen_layer(cfg, 0)
    q = gen_query(cfg, 0, peak=4.0)
    K = dense_from_logical(cfg, lay, bases["K"][0], "K")
    V = dense_from_logical(cfg, lay, bases["V"][0], "V")
    ref = sdpa_fp64(q, K, V, lay["n_tokens"], _alpha(cfg))
    got = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_random_basis_equals_sdpa_on_materialised_cache():
    cfg = tiny_config(seed=11, n_tokens=33, head_dim=32, r_max=16, resid_bits=4, resid_channels=4)
    bases = make_bases(cfg)
    lay = gen_layer(cfg, 1)
    q = gen_query(cfg, 1, peak=8.0)
    K = dense_from_logical(cfg, lay, bases["K"][0], "K")
    V = dense_from_logical(cfg, lay, bases["V"][0], "V")
    ref = sdpa_fp64(q, K, V, lay["n_tokens"], _alpha(cfg))
    got = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)
    assert rel_err(got, ref) <= 1e-12


def test_full_rank_zero_residual_is_attention_on_BC():
    """All tokens at full rank with no residual: exactly attention on
    K = C B, V = C_V B_V (the first invariant of the decode path)."""
    cfg = tiny_config(seed=5, n_tokens=20, head_dim=32, r_max=16, tier_rank=(16,), tier_prob=(1.0,),
                      resid_channels=0)
    bases = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    q = gen_query(cfg, 0, peak=3.0)
    K = np.einsum("bhnr,hrd->bhnd", lay["coefK"].astype(np.float64), bases["K"][0].astype(np.float64))
    V = np.einsum("bhnr,hrd->bhnd", lay["coefV"].astype(np.float64), bases["V"][0].astype(np.float64))
    ref = sdpa_fp64(q, K, V, lay["n_tokens"], _alpha(cfg))
    got = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)
    assert rel_err(got, ref) <= 1e-12


# ------------------------------------------------------------ closed forms
def _perm_setup(n, seed=3, s=2, d=16, r_max=8, tiers=(2, 4, 8)):
    cfg = tiny_config(batch=1, num_kv_heads=1, num_q_heads=2, head_dim=d, r_max=r_max,
                      tier_rank=tiers, tier_prob=(0.4, 0.3, 0.3), resid_channels=s, n_tokens=n,
                      seed=seed)
    bK, pK, sK = signed_permutation_basis(d, r_max, seed)
    bV, pV, sV = signed_permutation_basis(d, r_max, seed + 100)
    lay = gen_layer(cfg, 0)
    return cfg, lay, (bK, pK, sK), (bV, pV, sV)


def _vec_by_hand(cfg, lay, perm, sign, z, t):
    """Cached vector of token t written out: c_i * sign_i at channel perm_i,
    plus scale * value at each residual channel."""
    d = cfg.head_dim
    x = np.zeros(d)
    k = int(lay["tier"][0, 0, t])
    for i in range(cfg.tier_rank[k]):
        x[perm[i]] += sign[i] * float(lay["coef" + z][0, 0, t, i])
    for u in range(cfg.resid_per_tier[k]):
        x[int(lay["idx" + z][0, 0, t, u])] += float(lay["scale" + z][0, 0, t]) * float(lay["val" + z][0, 0, t, u])
    return x


def test_single_token_returns_its_value():
    cfg, lay, (bK, _, _), (bV, pV, sV) = _perm_setup(1)
    q = gen_query(cfg, 0, peak=5.0)
    got = oracle.decode(cfg, lay, bK[None], bV[None], q)
    v0 = _vec_by_hand(cfg, lay, pV, sV, "V", 0)
    for g in range(2):
        assert np.array_equal(got[0, g], v0)


def test_two_tokens_logistic_weights():
    cfg, lay, (bK, pK, sK), (bV, pV, sV) = _perm_setup(2, seed=9)
    q = gen_query(cfg, 0, peak=6.0)
    got = oracle.decode(cfg, lay, bK[None], bV[None], q)
    a = _alpha(cfg)
    k0, k1 = (_vec_by_hand(cfg, lay, pK, sK, "K", t) for t in (0, 1))
    v0, v1 = (_vec_by_hand(cfg, lay, pV, sV, "V", t) for t in (0, 1))
    for g in range(2):
        qq = q[0, g].astype(np.float64)
        dz = a * (qq @ k0 - qq @ k1)
        w0 = 1.0 / (1.0 + math.exp(-dz))
        ref = w0 * v0 + (1.0 - w0) * v1
        assert np.abs(got[0, g] - ref).max() <= 1e-14 * max(1.0, np.abs(ref).max())


def test_zero_query_gives_mean_value():
    cfg, lay, (bK, _, _), (bV, pV, sV) = _perm_setup(13, seed=21)
    q = np.zeros((1, 2, cfg.head_dim), np.float16)
    got = oracle.decode(cfg, lay, bK[None], bV[None], q)
    mean = np.mean([_vec_by_hand(cfg, lay, pV, sV, "V", t) for t in range(13)], axis=0)
    assert np.abs(got[0] - mean[None]).max() <= 1e-14


def test_constant_values_weights_sum_to_one():
    """Every token carries the same V: the output is that V for any query,
    which holds only if the softmax weights sum to one."""
    cfg, lay, (bK, _, _), (bV, pV, sV) = _perm_setup(40, seed=31)
    for key in ("coefV", "idxV", "valV", "scaleV"):
        lay[key][0, 0, :] = lay[key][0, 0, 0]
    lay["tier"][0, 0, :] = lay["tier"][0, 0, 0]
    q = gen_query(cfg, 0, peak=16.0)
    got = oracle.decode(cfg, lay, bK[None], bV[None], q)
    v0 = _vec_by_hand(cfg, lay, pV, sV, "V", 0)
    assert np.abs(got[0] - v0[None]).max() <= 1e-13 * max(1.0, np.abs(v0).max())


def test_zero_tokens_shrink_output_by_closed_form_ratio():
    """A token with zero coefficients and zero residual has logit exactly 0 and
    value 0.  With S = sum_t exp(z_t), adding one such token scales o by
    S/(S+1), two scale it by S/(S+2): (1/l2 - 1) == 2 (1/l1 - 1)."""
    cfg, lay, (bK, _, _), (bV, _, _) = _perm_setup(11, seed=41)
    q = gen_query(cfg, 0)
    o0 = oracle.decode(cfg, lay, bK[None], bV[None], q)
    outs = []
    for extra in (1, 2):
        lay2 = empty_layer(cfg, 11 + extra)
        for key in lay2:
            if key == "n_tokens":
                continue
            lay2[key][:, :, :11] = lay[key]
        outs.append(oracle.decode(cfg, lay2, bK[None], bV[None], q))
    for g in range(2):
        j = int(np.argmax(np.abs(o0[0, g])))
        l1 = outs[0][0, g] / o0[0, g, j]
        l2 = outs[1][0, g] / o0[0, g, j]
        lam1, lam2 = outs[0][0, g, j] / o0[0, g, j], outs[1][0, g, j] / o0[0, g, j]
        assert np.allclose(outs[0][0, g], lam1 * o0[0, g], rtol=0, atol=1e-15)
        assert np.allclose(outs[1][0, g], lam2 * o0[0, g], rtol=0, atol=1e-15)
        assert 0 < lam2 < lam1 < 1
        assert abs((1 / lam2 - 1) - 2 * (1 / lam1 - 1)) <= 1e-12 * (1 / lam2)


def test_empty_context_gives_zero():
    cfg = tiny_config()
    lay = empty_layer(cfg, 0)
    b = make_bases(cfg)
    got = oracle.decode(cfg, lay, b["K"][0], b["V"][0], gen_query(cfg, 0))
    assert np.array_equal(got, np.zeros_like(got))


def test_planted_needle_is_returned():
    """A needle whose logit leads every other token by >= 40 (natural log)
    makes the output its value to within n * e^-40 relative."""
    cfg, lay, (bK, pK, sK), (bV, pV, sV) = _perm_setup(300, seed=51)
    q = gen_query(cfg, 0)
    for pos in wg.needle_positions(300):
        lay2 = {k: v.copy() for k, v in lay.items()}
        wg.plant_needles(cfg, lay2, bK[None], q, [pos], lead=60.0)
        got = oracle.decode(cfg, lay2, bK[None], bV[None], q)
        kk = [_vec_by_hand(cfg, lay2, pK, sK, "K", t) for t in range(300)]
        z = np.array([_alpha(cfg) * (q[0, 0].astype(np.float64) @ k) for k in kk])
        assert z[pos] - np.max(np.delete(z, pos)) >= 40.0
        vn = _vec_by_hand(cfg, lay2, pV, sV, "V", pos)
        assert np.abs(got[0, 0] - vn).max() <= 300 * math.exp(-40) * np.abs(vn).max() + 1e-15


# ------------------------------------------------------------ invariants
def test_token_permutation_invariance():
    cfg = tiny_config(seed=61, n_tokens=50)
    b = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    q = gen_query(cfg, 0, peak=4.0)
    o = oracle.decode(cfg, lay, b["K"][0], b["V"][0], q)
    perm = np.random.default_rng(0).permutation(50)
    lay2 = {k: (v[:, :, perm].copy() if k != "n_tokens" else v) for k, v in lay.items()}
    o2 = oracle.decode(cfg, lay2, b["K"][0], b["V"][0], q)
    assert rel_err(o2, o) <= 1e-13


def test_value_linearity_doubles_exactly():
    cfg = tiny_config(seed=71, n_tokens=30)
    b = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    q = gen_query(cfg, 0)
    o = oracle.decode(cfg, lay, b["K"][0], b["V"][0], q)
    lay2 = dict(lay)
    lay2["coefV"] = (lay["coefV"].astype(np.float32) * 2).astype(np.float16)
    lay2["scaleV"] = (lay["scaleV"].astype(np.float32) * 2).astype(np.float16)
    o2 = oracle.decode(cfg, lay2, b["K"][0], b["V"][0], q)
    assert np.array_equal(o2, 2 * o)


def test_query_scale_tradeoff_is_exact():
    """Doubling q and halving the softmax scale leaves every logit unchanged."""
    cfg = tiny_config(seed=72, n_tokens=30)
    b = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    q = gen_query(cfg, 0)
    o = oracle.decode(cfg, lay, b["K"][0], b["V"][0], q, alpha=0.25)
    o2 = oracle.decode(cfg, lay, b["K"][0], b["V"][0], (q.astype(np.float32) * 2).astype(np.float16),
                       alpha=0.125)
    assert np.array_equal(o, o2)


def test_grouped_heads_and_batch_independence():
    cfg = tiny_config(seed=81, n_tokens=25)
    b = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    q = gen_query(cfg, 0)
    q[:, 1] = q[:, 0]            # heads 0 and 1 share KV head 0
    o = oracle.decode(cfg, lay, b["K"][0], b["V"][0], q)
    assert np.array_equal(o[:, 0], o[:, 1])
    assert not np.allclose(o[:, 0], o[:, 2])
    # changing sequence 1 leaves sequence 0 untouched
    lay2 = {k: v.copy() for k, v in lay.items()}
    lay2["coefV"][1] = 0
    o2 = oracle.decode(cfg, lay2, b["K"][0], b["V"][0], q)
    assert np.array_equal(o2[0], o[0]) and not np.array_equal(o2[1], o[1])


def test_pair_subset_matches_full_and_ragged_lengths():
    cfg = tiny_config(seed=91, n_tokens=40)
    b = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    lay["n_tokens"][:] = [40, 17]
    q = gen_query(cfg, 0)
    full = oracle.decode(cfg, lay, b["K"][0], b["V"][0], q)
    part = oracle.decode(cfg, lay, b["K"][0], b["V"][0], q, pairs=[(1, 1)])
    assert np.array_equal(part[1, 2:4], full[1, 2:4])
    assert np.isnan(part[0]).all()
    # the ragged sequence ignores tokens past its own length
    lay3 = {k: v.copy() for k, v in lay.items()}
    lay3["coefK"][1, :, 17:] = 7
    o3 = oracle.decode(cfg, lay3, b["K"][0], b["V"][0], q)
    assert np.array_equal(o3[1], full[1])
