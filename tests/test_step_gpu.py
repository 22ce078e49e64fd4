"""The one-launch decode step (dwkv_decode_step) against the two calls it
stands for and against the oracle (needs an MI355X).

dwkv_decode_step must leave the cache exactly as dwkv_decode_attn followed
by dwkv_append does: every byte of the exported layer, the slots and the
counts.  Its attention output equals theirs up to rounding: the step gives
the encoding workgroup a smaller share of the tiles, so the splits differ,
and each split rounds its probabilities to fp16 against its own running
max (2^-11 relative per term) -- within 1e-3 row-max normalised.  It is also checked on
its own: its output against the oracle's attention over the cache as it
stood before the step (2e-3 row-max normalised) and its appended token
against the oracle's encoding, bit for bit."""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases
from tests.helpers import extend_layer
from tests.test_append_gpu import _compare_token

pytestmark = pytest.mark.gpu

TOL = 2e-3
SAME = 1e-3     # fused step vs the two calls: another split of the tiles


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _steps(G, cfg, n0, steps, splits=0, gates=False, layer=1):
    import torch
    bases = make_bases(cfg)
    m = layer // cfg.layers_per_group
    caches = [G.make_cache(cfg, n=n0, extra=steps + 4, splits=splits) for _ in range(2)]
    sep, fused = caches
    try:
        lay = gen_layer(cfg, layer, n=n0)
        for c in caches:
            G.load_bases(c, bases, groups=[m])
            if n0 > 0:   # a new cache is empty
                G.load_layer(c, layer, lay)
        rng = np.random.default_rng(cfg.seed + 17)
        for step in range(steps):
            n = n0 + step
            q = gen_query(cfg, layer, step=step)
            a = gen_append_inputs(cfg, layer, step, bases)
            gk = gv = None
            if gates:
                gk = rng.choice([1.0, 0.5, 0.0], size=a["tier"].shape).astype(np.float16)
                gv = rng.choice([1.0, 0.25], size=a["tier"].shape).astype(np.float16)
            dgk = None if gk is None else G.dev(gk)
            dgv = None if gv is None else G.dev(gv)
            before = fused.read_counts(layer, cfg.batch)
            out_sep = sep.decode(layer, G.dev(q))
            sep.append(layer, G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"]), dgk, dgv)
            out_fused = fused.decode_step(layer, G.dev(q), G.dev(a["k"]), G.dev(a["v"]),
                                          G.dev(a["tier"]), dgk, dgv)
            torch.cuda.synchronize()
            got = out_fused.cpu().numpy()
            if n > 0:
                same = G.norm_err(got.astype(np.float64), out_sep.cpu().numpy().astype(np.float64))
                assert same.max() <= SAME, f"step {step}: output differs from decode + append"
            else:
                assert not got.any() and not out_sep.cpu().numpy().any()
            ex_s, cnt_s, sl_s = G.export_np(sep, layer, cfg.batch, n + 1)
            ex_f, cnt_f, sl_f = G.export_np(fused, layer, cfg.batch, n + 1)
            assert np.array_equal(cnt_s, cnt_f) and np.array_equal(sl_s, sl_f)
            for key in ex_s:
                assert np.array_equal(ex_s[key].view(np.uint8), ex_f[key].view(np.uint8)), key
            ref = oracle.decode(cfg, lay, bases["K"][m], bases["V"][m], q)
            if n == 0:
                assert not got.any()
            else:
                err = G.norm_err(got.astype(np.float64), ref)
                assert err.max() <= TOL, f"step {step}: max normalised error {err.max():.3e}"
            enc = oracle.append_layer(cfg, bases["K"][m], bases["V"][m], a["k"], a["v"], a["tier"],
                                      gateK=gk, gateV=gv)
            _compare_token(cfg, ex_f, sl_f, before, n, enc, a["tier"])
            lay = extend_layer(lay, enc, a["tier"], n)
        for c in caches:
            assert c.check_errors() == 0
    finally:
        for c in caches:
            c.close()


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_step_tiny_reference(G, splits):
    _steps(G, w.get_config(0), w.get_config(0).n_tokens, steps=6, splits=splits)


def test_step_with_gates(G):
    _steps(G, w.get_config(0), 700, steps=4, gates=True)


def test_step_llama8b_shape_batched(G):
    cfg = w.get_config(1).with_(batch=3)
    _steps(G, cfg, 1500, steps=3, layer=5)


def test_step_batch16_router_skew(G):
    cfg = w.get_config(3)
    _steps(G, cfg, 600, steps=2, layer=2)


def test_step_llama70b_shape(G):
    cfg = w.get_config(4)
    _steps(G, cfg, 900, steps=2, layer=7)


def test_step_on_empty_cache(G):
    """An empty cache: zero output, and the step's token becomes the first."""
    cfg = w.get_config(0)
    _steps(G, cfg, 0, steps=3)


def test_step_full_tier_sets_error_and_keeps_output(G):
    """Forced from the host: a full top tier.  The step still attends over
    the cache, sets the error word and drops the token, like dwkv_append."""
    import compressed_kv_cache_dwkv_amd as d
    cfg = w.get_config(0)
    bases = make_bases(cfg)
    lay = gen_layer(cfg, 0)
    top = cfg.num_tiers - 1
    full = int((lay["tier"][0, 0] == top).sum())
    from workload.gen import max_tier_counts
    cap = [int(c) + 4 for c in max_tier_counts(cfg)]
    cap[top] = full
    cache = G.make_cache(cfg, capacity=cap, extra=8)
    try:
        G.load_bases(cache, bases)
        G.load_layer(cache, 0, lay)
        assert cache.check_errors() == 0
        q = gen_query(cfg, 0)
        a = gen_append_inputs(cfg, 0, 0, bases)
        tier = np.full(a["tier"].shape, top, np.uint8)
        before = cache.read_counts(0, cfg.batch)
        out = cache.decode_step(0, G.dev(q), G.dev(a["k"]), G.dev(a["v"]), G.dev(tier))
        bits = cache.check_errors()
        assert bits & d.DWKV_DEVERR_TIER_FULL
        assert np.array_equal(cache.read_counts(0, cfg.batch), before)
        ref = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)
        assert G.norm_err(out.cpu().numpy().astype(np.float64), ref).max() <= TOL
    finally:
        cache.close()
