"""GPU append against the CPU oracle, bit for bit (needs an MI355X).

The appended token's tier, its slot (= tokens already in the tier), every
coefficient bit, the kept channel indices, every code and the scale bits
must equal the oracle's encoding of the same fp16 input."""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases
from tests.helpers import extend_layer, tiny_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _compare_token(cfg, exported, slots, counts_before, pos, enc, tier):
    B, H = tier.shape
    for b in range(B):
        for h in range(H):
            k = int(tier[b, h])
            assert exported["tier"][b, h, pos] == k
            assert slots[b, h, pos] == counts_before[b, h, k], "slot must be the tier's old count"
            r, s = cfg.tier_rank[k], cfg.resid_per_tier[k]
            for z in "KV":
                got_c = exported["coef" + z][b, h, pos]
                ref_c = enc["coef" + z][b, h]
                got_c = got_c.view(np.uint16) if got_c.dtype == np.float16 else got_c.view(np.uint8)
                ref_c = ref_c.view(np.uint16) if ref_c.dtype == np.float16 else ref_c.view(np.uint8)
                assert np.array_equal(got_c[:r], ref_c[:r]), f"coef{z} (b={b},h={h})"
                assert not got_c[r:].any()
                if "cscale" + z in enc:
                    assert exported["cscale" + z][b, h, pos].view(np.uint16) == \
                        enc["cscale" + z][b, h].view(np.uint16), f"cscale{z}"
                assert np.array_equal(exported["idx" + z][b, h, pos, :s], enc["idx" + z][b, h, :s])
                assert np.array_equal(exported["val" + z][b, h, pos, :s], enc["val" + z][b, h, :s])
                if s > 0:
                    assert exported["scale" + z][b, h, pos].view(np.uint16) == \
                        enc["scale" + z][b, h].view(np.uint16), f"scale{z}"


def _append_steps(G, cfg, steps, n0=None, gates=False, bases=None, layer=0):
    import torch
    bases = make_bases(cfg) if bases is None else bases
    n0 = cfg.n_tokens if n0 is None else n0
    cache = G.make_cache(cfg, n=n0, extra=steps + 4)
    m = layer // cfg.layers_per_group
    try:
        G.load_bases(cache, bases, groups=[m])
        lay = gen_layer(cfg, layer, n=n0)
        G.load_layer(cache, layer, lay)
        rng = np.random.default_rng(cfg.seed + 5)
        for step in range(steps):
            before = cache.read_counts(layer, cfg.batch)
            a = gen_append_inputs(cfg, layer, step, bases)
            gk = gv = None
            if gates:
                gk = rng.choice([1.0, 0.5, 0.3, 0.0], size=a["tier"].shape).astype(np.float16)
                gv = rng.choice([1.0, 0.75, 0.1], size=a["tier"].shape).astype(np.float16)
            cache.append(layer, G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"]),
                         None if gk is None else G.dev(gk), None if gv is None else G.dev(gv))
            enc = oracle.append_layer(cfg, bases["K"][m], bases["V"][m], a["k"], a["v"], a["tier"],
                                      gateK=gk, gateV=gv)
            exported, counts, slots = G.export_np(cache, layer, cfg.batch, n0 + steps)
            _compare_token(cfg, exported, slots, before, n0 + step, enc, a["tier"])
            after = cache.read_counts(layer, cfg.batch)
            delta = after - before
            for b in range(cfg.batch):
                for h in range(cfg.num_kv_heads):
                    exp = np.zeros(cfg.num_tiers, np.int32)
                    exp[int(a["tier"][b, h])] = 1
                    assert np.array_equal(delta[b, h], exp)
        assert cache.check_errors() == 0
        return cache, bases, lay
    except Exception:
        cache.close()
        raise


def test_import_export_round_trip(G):
    cfg = w.get_config(1).with_(batch=2)
    bases = make_bases(cfg)
    cache = G.make_cache(cfg, n=5000)
    try:
        G.load_bases(cache, bases, groups=[0])
        lay = gen_layer(cfg, 1, n=5000)
        lay["n_tokens"][:] = [5000, 3333]
        G.load_layer(cache, 1, lay)
        ex, counts, slots = G.export_np(cache, 1, 2, 5000)
        for b, n in ((0, 5000), (1, 3333)):
            for key in ("tier", "coefK", "coefV", "idxK", "idxV", "valK", "valV", "scaleK", "scaleV"):
                assert np.array_equal(ex[key][b, :, :n].view(np.uint8), lay[key][b, :, :n].view(np.uint8)), key
            for h in range(cfg.num_kv_heads):
                t = lay["tier"][b, h, :n]
                assert np.array_equal(counts[b, h], np.bincount(t, minlength=cfg.num_tiers))
                for k in range(cfg.num_tiers):   # slots follow position order inside a tier
                    assert np.array_equal(slots[b, h, :n][t == k], np.arange((t == k).sum()))
        assert cache.check_errors() == 0
    finally:
        cache.close()


@pytest.mark.parametrize("ci", [0, 1])
def test_append_bit_exact(G, ci):
    cfg = w.get_config(ci)
    cfg = cfg.with_(batch=4) if ci == 1 else cfg
    cache, _, _ = _append_steps(G, cfg, steps=6, n0=300)
    cache.close()


def test_append_with_gates_and_int8(G):
    cfg = tiny_config(batch=3, num_q_heads=8, num_kv_heads=4, head_dim=128, r_max=64,
                      tier_rank=(8, 16, 32, 64), tier_prob=(0.25, 0.25, 0.25, 0.25),
                      resid_channels=6, resid_bits=8, n_tokens=100)
    cache, _, _ = _append_steps(G, cfg, steps=4, n0=50, gates=True)
    cache.close()


def test_append_paper_literal_tiers(G):
    """Fixed coefficient width with routed residual channels 0/2/4/8 (the
    rank levels the paper's router uses), 4-bit codes."""
    cfg = tiny_config(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, r_max=32,
                      tier_rank=(4, 8, 16, 32), tier_prob=(0.25, 0.25, 0.25, 0.25),
                      tier_resid=(0, 2, 4, 8), resid_channels=8, resid_bits=4, n_tokens=64)
    cache, _, _ = _append_steps(G, cfg, steps=5, n0=64)
    cache.close()


@pytest.mark.parametrize("ci", [0, 1])
def test_append_bit_exact_8bit_coefficients(G, ci):
    """The 8-bit blockwise coefficient form: codes, block scale, kept
    channels, residual codes and scale, bit for bit."""
    cfg = w.get_config(ci).with_(coef_bits=8)
    cfg = cfg.with_(batch=16) if ci == 1 else cfg
    cache, _, _ = _append_steps(G, cfg, steps=6, n0=200, gates=ci == 1)
    cache.close()


def test_import_export_round_trip_8bit_coefficients(G):
    cfg = w.get_config(1).with_(batch=2, coef_bits=8)
    bases = make_bases(cfg)
    cache = G.make_cache(cfg, n=3000)
    try:
        G.load_bases(cache, bases, groups=[0])
        lay = gen_layer(cfg, 1, n=3000)
        lay["n_tokens"][:] = [3000, 1111]
        G.load_layer(cache, 1, lay)
        ex, counts, slots = G.export_np(cache, 1, 2, 3000)
        for b, n in ((0, 3000), (1, 1111)):
            for key in ("tier", "coefK", "coefV", "cscaleK", "cscaleV", "idxK", "idxV", "valK", "valV", "scaleK",
                        "scaleV"):
                assert np.array_equal(ex[key][b, :, :n].view(np.uint8), lay[key][b, :, :n].view(np.uint8)), key
        assert cache.check_errors() == 0
    finally:
        cache.close()


def test_append_many_random_vectors(G):
    """102,400 encodings (256 sequences x 8 heads x 2 (K,V) x 25 steps) of
    the Llama-3-8B shape, each bit for bit."""
    cfg = w.get_config(1).with_(batch=256)
    cache, _, _ = _append_steps(G, cfg, steps=25, n0=8)
    cache.close()


def _append_given(G, cfg, bases, k, v, tier, n0=4):
    """One append of the given fp16 vectors k, v [B][H][d] and tiers, compared
    bit for bit with the oracle's encoding."""
    cache = G.make_cache(cfg, n=n0, extra=4)
    try:
        G.load_bases(cache, bases, groups=[0])
        lay = gen_layer(cfg, 0, n=n0)
        G.load_layer(cache, 0, lay)
        before = cache.read_counts(0, cfg.batch)
        cache.append(0, G.dev(k), G.dev(v), G.dev(tier))
        enc = oracle.append_layer(cfg, bases["K"][0], bases["V"][0], k, v, tier)
        exported, counts, slots = G.export_np(cache, 0, cfg.batch, n0 + 1)
        _compare_token(cfg, exported, slots, before, n0, enc, tier)
        assert cache.check_errors() == 0
        return enc
    finally:
        cache.close()


@pytest.mark.parametrize("bits", [4, 8])
def test_append_planted_ties(G, bits):
    """Identity bases and inputs drawn from a handful of values, so most
    residual magnitudes tie with others: the kept channels must follow the
    tie rule (larger |e| first, then the smaller channel) on the GPU too."""
    d = 64
    cfg = tiny_config(batch=48, num_q_heads=4, num_kv_heads=2, head_dim=d, r_max=d,
                      tier_rank=(8, 16, 32, 64), tier_prob=(0.25, 0.25, 0.25, 0.25),
                      resid_channels=8 if bits == 4 else 5, resid_bits=bits, n_tokens=4)
    bases = make_bases(cfg, identity=True)
    rng = np.random.default_rng(71 + bits)
    vals = np.array([0.0, 0.25, -0.25, 0.5, -0.5, 1.0, -1.0], np.float16)
    B, H = cfg.batch, cfg.num_kv_heads
    k = vals[rng.integers(0, len(vals), size=(B, H, d))]
    v = vals[rng.integers(0, len(vals), size=(B, H, d))]
    tier = rng.integers(0, 3, size=(B, H)).astype(np.uint8)       # ranks 8..32: residual channels remain
    enc = _append_given(G, cfg, bases, k, v, tier)
    # the ties really are there: some kept channel ties with an unkept one
    tied = 0
    for b in range(B):
        for h in range(H):
            r = cfg.tier_rank[int(tier[b, h])]
            e = np.abs(k[b, h].astype(np.float32))
            e[:r] = 0.0                                      # B = I: e is x past the rank
            kept = enc["idxK"][b, h, :cfg.resid_channels].astype(int)
            low = e[kept].min()
            tied += int((e[np.setdiff1d(np.arange(d), kept)] == low).any())
    assert tied > B * H // 4


def test_append_in_span_vectors_have_zero_scale(G):
    """Vectors inside the span of the first r basis vectors of exact bases
    (identity and signed-permutation): the residual is exactly zero, so the
    scale and every code are 0 and the kept channels are 0..s-1."""
    from tests.helpers import signed_permutation_basis
    d, R = 128, 64
    cfg = tiny_config(batch=16, num_q_heads=8, num_kv_heads=2, head_dim=d, r_max=R,
                      tier_rank=(8, 16, 32, 64), tier_prob=(0.25, 0.25, 0.25, 0.25),
                      resid_channels=8, resid_bits=4, n_tokens=4)
    rng = np.random.default_rng(5)
    B, H = cfg.batch, cfg.num_kv_heads
    for kind in ("identity", "permutation"):
        if kind == "identity":
            bases = {"K": np.zeros((1, H, R, d), np.float16), "V": np.zeros((1, H, R, d), np.float16)}
            for z in "KV":
                bases[z][0, :] = np.eye(d, dtype=np.float16)[:R]
        else:
            bases = {"K": np.zeros((1, H, R, d), np.float16), "V": np.zeros((1, H, R, d), np.float16)}
            for zi, z in enumerate("KV"):
                for h in range(H):
                    bases[z][0, h] = signed_permutation_basis(d, R, 10 * zi + h)[0]
        tier = rng.integers(0, 4, size=(B, H)).astype(np.uint8)
        k = np.zeros((B, H, d), np.float16)
        v = np.zeros((B, H, d), np.float16)
        for b in range(B):
            for h in range(H):
                r = cfg.tier_rank[int(tier[b, h])]
                for x, z in ((k, "K"), (v, "V")):
                    c = rng.standard_normal(r).astype(np.float16)
                    x[b, h] = (c.astype(np.float32) @ bases[z][0, h, :r].astype(np.float32)).astype(np.float16)
        enc = _append_given(G, cfg, bases, k, v, tier)
        for z in "KV":
            assert not enc["scale" + z].view(np.uint16).any()
            assert not enc["val" + z].any()
            assert (enc["idx" + z] == np.arange(8, dtype=np.uint8)).all()


def test_identity_basis_append_is_hand_predictable(G):
    """B = I: coefficients are the first r inputs, kept channels the largest
    remaining |x_j|."""
    cfg = tiny_config(batch=1, num_q_heads=2, num_kv_heads=1, head_dim=64, r_max=64,
                      tier_rank=(8, 64), tier_prob=(1.0, 0.0), resid_channels=4, resid_bits=4,
                      n_tokens=4)
    bases = make_bases(cfg, identity=True)
    cache, _, _ = _append_steps(G, cfg, steps=3, n0=4, bases=bases)
    try:
        ex, _, _ = G.export_np(cache, 0, 1, 7)
        a = gen_append_inputs(cfg, 0, 0, bases)
        x = a["k"][0, 0]
        t = int(a["tier"][0, 0])
        r = cfg.tier_rank[t]
        assert np.array_equal(ex["coefK"][0, 0, 4, :r].view(np.uint16), x[:r].view(np.uint16))
        if r < 64:
            tail = np.abs(x[r:].astype(np.float32))
            order = sorted(range(64 - r), key=lambda j: (-tail[j], j))[:4]
            assert list(ex["idxK"][0, 0, 4, :4]) == sorted(j + r for j in order)
    finally:
        cache.close()


def test_attend_then_append_and_append_then_attend(G):
    """Both orders of the decode procedure match the oracle on the cache they
    see: before the append (the new token absent) and after it (present)."""
    cfg = w.get_config(0)
    bases = make_bases(cfg)
    cache = G.make_cache(cfg, extra=8)
    try:
        G.load_bases(cache, bases)
        lay = gen_layer(cfg, 1)
        G.load_layer(cache, 1, lay)
        q = gen_query(cfg, 1, step=3)
        ref0 = oracle.decode(cfg, lay, bases["K"][0], bases["V"][0], q)
        got0 = G.decode_np(cache, 1, q)
        assert G.norm_err(got0, ref0).max() <= 2e-3
        a = gen_append_inputs(cfg, 1, 0, bases)
        cache.append(1, G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"]))
        got1 = G.decode_np(cache, 1, q)
        enc = oracle.append_layer(cfg, bases["K"][0], bases["V"][0], a["k"], a["v"], a["tier"])
        n = cfg.n_tokens
        lay2 = extend_layer(lay, enc, a["tier"], n)
        ref1 = oracle.decode(cfg, lay2, bases["K"][0], bases["V"][0], q)
        assert G.norm_err(got1, ref1).max() <= 2e-3
        assert not np.allclose(ref0, ref1)
    finally:
        cache.close()


def test_full_tier_sets_device_error_and_drops_token(G):
    """Forced from the host: a tier capacity equal to the tokens already in
    it makes the next append of that tier set the error word."""
    cfg = w.get_config(0)
    bases = make_bases(cfg)
    from workload.gen import max_tier_counts
    cap = [int(c) for c in max_tier_counts(cfg)]
    cache = G.make_cache(cfg, capacity=[c + 4 for c in cap[:-1]] + [cap[-1]], extra=8)
    try:
        G.load_bases(cache, bases)
        lay = gen_layer(cfg, 0)
        G.load_layer(cache, 0, lay)
        full = int((lay["tier"][0, 0] == 3).sum())
        cache.clear_errors()
        tier = np.full((1, 1), 3, np.uint8)
        a = gen_append_inputs(cfg, 0, 0, bases)
        before = cache.read_counts(0, 1)
        cache.append(0, G.dev(a["k"]), G.dev(a["v"]), G.dev(tier))
        bits = cache.check_errors()
        if full == cap[-1]:
            import compressed_kv_cache_dwkv_amd as d
            assert bits & d.DWKV_DEVERR_TIER_FULL
            assert np.array_equal(cache.read_counts(0, 1), before)
        cache.clear_errors()
        assert cache.check_errors() == 0
        tier[:] = 7   # not a tier
        cache.append(0, G.dev(a["k"]), G.dev(a["v"]), G.dev(tier))
        import compressed_kv_cache_dwkv_amd as d
        assert cache.check_errors() & d.DWKV_DEVERR_BAD_TIER
    finally:
        cache.close()
