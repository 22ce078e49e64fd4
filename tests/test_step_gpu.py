"""The one-launch decode step (dwkv_decode_step) against the two calls it
stands for and against the oracle (needs an MI355X).

dwkv_decode_step must leave the cache exactly as dwkv_decode_attn followed
by dwkv_append does: every byte of the exported layer, the slots and the
counts.  Its output is checked against the oracle's attention over the
cache as it stood before the step (2e-3 row-max normalised) and its appended
token against the oracle's encoding, bit for bit.  Its output also equals the
two calls' up to rounding, held to the same 2e-3: the step gives the
encoding workgroup a smaller share of the tiles, so the splits differ, and
each split rounds its probabilities to fp16 against its own running max
(relative error up to 2^-11 per term).  Near-uniform attention over a short
context averages those independent roundings down the least: at 600
tokens the two forms differ by up to about 1e-3 of the row max."""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases
from tests.helpers import extend_layer
from tests.test_append_gpu import _compare_token

pytestmark = pytest.mark.gpu

TOL = 2e-3
SAME = TOL      # fused step vs the two calls: another split of the tiles


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _steps(G, cfg, n0, steps, splits=0, gates=False, layer=1, expect_splits=None):
    import torch
    bases = make_bases(cfg)
    m = layer // cfg.layers_per_group
    caches = [G.make_cache(cfg, n=n0, extra=steps + 4, splits=splits) for _ in range(2)]
    sep, fused = caches
    try:
        print(f"step test: {cfg.name} n0={n0} layer={layer} splits={fused.splits}", flush=True)
        if expect_splits is not None:
            assert fused.splits == expect_splits
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
            ref = oracle.decode(cfg, lay, bases["K"][m], bases["V"][m], q)
            if n > 0:
                err = G.norm_err(got.astype(np.float64), ref)
                assert err.max() <= TOL, f"step {step}: max normalised error {err.max():.3e}"
                err_sep = G.norm_err(out_sep.cpu().numpy().astype(np.float64), ref)
                assert err_sep.max() <= TOL, f"step {step}: two-call error {err_sep.max():.3e}"
                same = G.norm_err(got.astype(np.float64), out_sep.cpu().numpy().astype(np.float64))
                assert same.max() <= SAME, f"step {step}: output differs from decode + append"
                print(f"  step {step}: error {err.max():.2e}, two calls {err_sep.max():.2e}, "
                      f"between them {same.max():.2e}", flush=True)
            else:
                assert not got.any() and not out_sep.cpu().numpy().any()
            ex_s, cnt_s, sl_s = G.export_np(sep, layer, cfg.batch, n + 1)
            ex_f, cnt_f, sl_f = G.export_np(fused, layer, cfg.batch, n + 1)
            assert np.array_equal(cnt_s, cnt_f) and np.array_equal(sl_s, sl_f)
            for key in ex_s:
                assert np.array_equal(ex_s[key].view(np.uint8), ex_f[key].view(np.uint8)), key
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


# (splits 0 = the automatic count, which is 1 for these short caches; 8 and
# 32 put most of the fixed first tiles past tier 0's tokens and move every
# split boundary by the encoder's share)
@pytest.mark.parametrize("splits", [0, 8, 32])
def test_step_llama8b_shape_batched(G, splits):
    cfg = w.get_config(1).with_(batch=3)
    _steps(G, cfg, 1500, steps=3, layer=5, splits=splits)


# (2 and 3 splits: the encoding share of a launch with at most 4 splits
# per head, the full-size 32K x 16 workload's case)
@pytest.mark.parametrize("splits", [0, 2, 3, 8, 32])
def test_step_batch16_router_skew(G, splits):
    cfg = w.get_config(3)
    _steps(G, cfg, 600, steps=2, layer=2, splits=splits)


@pytest.mark.parametrize("splits", [0, 3, 8, 32])
def test_step_llama70b_shape(G, splits):
    cfg = w.get_config(4)
    _steps(G, cfg, 900, steps=2, layer=7, splits=splits)


@pytest.mark.parametrize("ci,layer", [(2, 13), (4, 41)])
def test_step_full_size_as_benchmarked(G, ci, layer):
    """The launch the benchmark times: dwkv_decode_step at the workload's
    full context (64K Llama-3-8B shape, 128K Llama-3-70B shape with 8 query
    heads per KV head) and the automatic split count (32), two steps.  Every
    KV head's output against the oracle over the cache before the step, the
    appended tokens bit for bit, the output against the two calls, and the
    whole layer byte for byte against the two calls' cache."""
    cfg = w.get_config(ci)
    _steps(G, cfg, cfg.n_tokens, steps=2, layer=layer, expect_splits=32)


def test_step_paper_literal_tiers(G):
    """Fixed coefficient width r_b = 32 with routed residual channels 0/2/4/8:
    the one-launch step against the two calls and the oracle."""
    from tests.helpers import tiny_config
    cfg = tiny_config(batch=2, num_layers=4, layers_per_group=2, num_kv_heads=4, num_q_heads=16, head_dim=128,
                      r_max=32, tier_rank=(32,) * 4, tier_prob=(0.4, 0.3, 0.2, 0.1), tier_resid=(0, 2, 4, 8),
                      resid_channels=8, resid_bits=4, n_tokens=1800)
    _steps(G, cfg, 1800, steps=3, layer=3, splits=4)


@pytest.mark.parametrize("ci,n0,splits", [(0, 1024, 3), (1, 1500, 8), (2, 65536, 0)])
def test_step_8bit_coefficients(G, ci, n0, splits):
    """The one-launch step with 8-bit blockwise coefficients (the encoder
    quantises the new token's coefficients in the same launch)."""
    cfg = w.get_config(ci).with_(coef_bits=8)
    _steps(G, cfg, n0, steps=2, layer=1, splits=splits)


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


def _extend_ragged(lay: dict, enc: dict, tier: np.ndarray) -> dict:
    """`lay` with the oracle's encoding of one token per (b, KV head) put at
    each sequence's own next position (sequences of different lengths)."""
    ns = lay["n_tokens"].astype(np.int64)
    need = int(ns.max()) + 1
    out = {}
    for key, v in lay.items():
        if key == "n_tokens":
            out[key] = ns + 1
            continue
        shape = list(v.shape)
        shape[2] = max(shape[2], need)
        nv = np.zeros(shape, v.dtype)
        nv[:, :, :v.shape[2]] = v
        out[key] = nv
    for b, n in enumerate(ns):
        out["tier"][b, :, n] = tier[b]
        for z in "KV":
            for f in ("coef", "idx", "val", "scale", "cscale"):
                if f + z in enc:
                    out[f + z][b, :, n] = enc[f + z][b]
    return out


def test_step_ragged_batch_with_empty_and_one_token_sequences(G):
    """One-launch steps on a batch whose sequences hold 0, 1 and 3000 tokens,
    at 32 splits per KV head: most workgroups of the short sequences have no
    tile (their splits publish empty partials), the empty sequence's first
    output is exactly zero, and every sequence's token goes to its own next
    position.  Three steps, each against the oracle over the cache before it
    and against decode + append on a twin cache (outputs within the bound,
    the layer byte for byte); the appended tokens bit for bit."""
    import torch
    cfg = w.get_config(1).with_(batch=3)
    layer, steps, ns0 = 6, 3, [0, 1, 3000]
    bases = make_bases(cfg)
    m = layer // cfg.layers_per_group
    caches = [G.make_cache(cfg, n=max(ns0), extra=steps + 4, splits=32) for _ in range(2)]
    sep, fused = caches
    try:
        print(f"ragged step test: {cfg.name} lengths={ns0} splits={fused.splits}", flush=True)
        assert fused.splits == 32
        lay = gen_layer(cfg, layer, n=max(ns0))
        lay["n_tokens"][:] = ns0
        for c in caches:
            G.load_bases(c, bases, groups=[m])
            G.load_layer(c, layer, lay)
        for step in range(steps):
            ns = [int(x) for x in lay["n_tokens"]]
            q = gen_query(cfg, layer, step=step)
            a = gen_append_inputs(cfg, layer, step, bases)
            before = fused.read_counts(layer, cfg.batch)
            assert np.array_equal(before.sum(axis=-1), np.array(ns)[:, None].repeat(cfg.num_kv_heads, 1))
            out_sep = sep.decode(layer, G.dev(q))
            sep.append(layer, G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"]))
            out_fused = fused.decode_step(layer, G.dev(q), G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"]))
            torch.cuda.synchronize()
            got, two = out_fused.cpu().numpy(), out_sep.cpu().numpy()
            ref = oracle.decode(cfg, lay, bases["K"][m], bases["V"][m], q)
            live = np.array(ns) > 0
            for b in np.nonzero(~live)[0]:
                assert not got[b].any() and not two[b].any(), f"step {step}: empty sequence {b} must give 0"
            err = G.norm_err(got.astype(np.float64), ref)[live]
            err_sep = G.norm_err(two.astype(np.float64), ref)[live]
            same = G.norm_err(got.astype(np.float64), two.astype(np.float64))[live]
            assert err.max() <= TOL, f"step {step}: max normalised error {err.max():.3e}"
            assert err_sep.max() <= TOL and same.max() <= SAME
            print(f"  step {step} lengths {ns}: error {err.max():.2e}, two calls {err_sep.max():.2e}", flush=True)
            n_max = max(ns) + 1
            ex_s, cnt_s, sl_s = G.export_np(sep, layer, cfg.batch, n_max)
            ex_f, cnt_f, sl_f = G.export_np(fused, layer, cfg.batch, n_max)
            assert np.array_equal(cnt_s, cnt_f) and np.array_equal(sl_s, sl_f)
            for key in ex_s:
                assert np.array_equal(ex_s[key].view(np.uint8), ex_f[key].view(np.uint8)), key
            enc = oracle.append_layer(cfg, bases["K"][m], bases["V"][m], a["k"], a["v"], a["tier"])
            for b in range(cfg.batch):
                _compare_token(cfg.with_(batch=1), {k: v[b:b + 1] for k, v in ex_f.items()}, sl_f[b:b + 1],
                               before[b:b + 1], ns[b], {k: v[b:b + 1] for k, v in enc.items()}, a["tier"][b:b + 1])
            lay = _extend_ragged(lay, enc, a["tier"])
        for c in caches:
            assert c.check_errors() == 0
    finally:
        for c in caches:
            c.close()
