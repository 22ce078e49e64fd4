"""Pins of oracle.probe_error (the paper's Eq. (3)) and oracle.probe_controller
(the threshold feedback described after Eq. (3)) on the CPU."""
import numpy as np
import pytest

import oracle
from workload.gen import gen_layer, gen_query, make_bases
from tests.helpers import tiny_config


def _exact_cfg():
    # B = I with r = d and no residual: the compressed cache holds K, V exactly
    return tiny_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=16, r_max=16, tier_rank=(16,),
                       tier_prob=(1.0,), tier_resid=(0,), resid_channels=0, resid_bits=4, n_tokens=30)


def test_probe_error_is_zero_when_the_reference_is_the_cache():
    cfg = _exact_cfg()
    bases = make_bases(cfg, identity=True)
    lay = gen_layer(cfg, 0)
    K, V = lay["coefK"].copy(), lay["coefV"].copy()          # exactly K^, V^ (fp16)
    qs = [gen_query(cfg, 0, step=i) for i in range(3)]
    e = oracle.probe_error(cfg, lay, bases["K"][0], bases["V"][0], K, V, lay["n_tokens"], qs)
    assert e.max() <= 1e-13


def test_probe_error_closed_form_for_scaled_values():
    """Reference values twice the cache's: Attn doubles, so e = ||2o - o|| / ||2o|| = 1/2."""
    cfg = _exact_cfg()
    bases = make_bases(cfg, identity=True)
    lay = gen_layer(cfg, 0)
    K, V = lay["coefK"].copy(), (lay["coefV"].astype(np.float32) * 2).astype(np.float16)
    qs = [gen_query(cfg, 0, step=i) for i in range(2)]
    e = oracle.probe_error(cfg, lay, bases["K"][0], bases["V"][0], K, V, lay["n_tokens"], qs, eps=0.0)
    assert np.abs(e - 0.5).max() <= 1e-13


def test_probe_error_norm_runs_over_positions_and_heads():
    """Against a direct NumPy evaluation of Eq. (3) from the two pinned
    attention oracles, on a general cache with a perturbed reference."""
    cfg = tiny_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=32, r_max=16, tier_rank=(4, 8, 16),
                      tier_prob=(0.5, 0.3, 0.2), resid_channels=3, resid_bits=4, n_tokens=40)
    bases = make_bases(cfg)
    lay = gen_layer(cfg, 1)
    K, V = oracle.materialize(cfg, lay, bases["K"][0], bases["V"][0])
    rng = np.random.default_rng(4)
    K = (K + 0.05 * rng.standard_normal(K.shape)).astype(np.float16)
    V = (V + 0.05 * rng.standard_normal(V.shape)).astype(np.float16)
    qs = [gen_query(cfg, 1, step=i) for i in range(4)]
    e = oracle.probe_error(cfg, lay, bases["K"][0], bases["V"][0], K, V, lay["n_tokens"], qs, eps=1e-6)
    for b in range(2):
        for h in range(2):
            diff = ref = 0.0
            for q in qs:
                oe = oracle.dense_decode(K, V, lay["n_tokens"], q)[b, 4 * h:4 * h + 4]
                oc = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)[b, 4 * h:4 * h + 4]
                diff += float(((oe - oc) ** 2).sum())
                ref += float((oe ** 2).sum())
            assert abs(e[b, h] - np.sqrt(diff) / (np.sqrt(ref) + 1e-6)) <= 1e-12
    assert e.min() > 0.01


def test_probe_controller_trajectory_by_hand():
    """tol 0.03, step 0.05, patience 3, tau in [0, 1]: an error above the
    tolerance lowers tau at once; three intervals below raise it."""
    tau, below = 0.5, 0
    seq = [0.01, 0.02, 0.01, 0.05, 0.01, 0.01, 0.02, 0.02, 0.01, 0.01]
    taus = []
    for e in seq:
        tau, below = oracle.probe_controller(tau, below, e, 0.03, 0.05, 3, 0.0, 1.0)
        taus.append(round(tau, 6))
    assert taus == [0.5, 0.5, 0.55, 0.5, 0.5, 0.5, 0.55, 0.55, 0.55, 0.6]
    # clamps
    t, _ = oracle.probe_controller(0.02, 0, 1.0, 0.03, 0.05, 3, 0.0, 1.0)
    assert t == 0.0
    t, _ = oracle.probe_controller(0.98, 2, 0.0, 0.03, 0.05, 3, 0.0, 1.0)
    assert t == 1.0
