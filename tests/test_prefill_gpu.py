"""Prefill compression through the C ABI against the oracle (needs an MI355X).

  * Gram sums: bit-exact on integer-valued prefill data (every product and
    partial sum is an integer below 2^24, exact in fp32 in any order), and
    within the fp32 summation bound |dC_ij| <= m 2^-24 sum_t |x_ti x_tj|
    (m: vectors one workgroup sums, at most a layer's) on Gaussian data,
    whose tail positions hold NaN (they must not count).
  * Bases: on identical Gram matrices (the integer data) the Ritz values
    agree to 1e-10 of the largest, and each basis row whose Ritz value is
    separated from its neighbours by 1e-6 of the largest is the oracle's fp64
    row rounded once to fp16 (within half an fp16 unit plus 1e-9).  On
    Gaussian data the difference of the two Gram matrices dC enters
    (Weyl: Ritz values within 2 ||dC||_2; Davis-Kahan: converged rows within
    2 sqrt(2) ||dC||_2 / gap).
  * Bulk encode: bit-exact against the oracle (every token exactly one
    append) given the same seeded bases, for fp16 and 8-bit coefficients,
    head_dim 64 and 128, gates, ragged lengths, paper-literal tiers, and in
    two chunks; refusals leave a (sequence, KV head) unchanged.
  * The three steps in a chain, and the full 64K-token Llama-3-8B shape.
"""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_gates, gen_prefill, gen_query, gen_sketch, gen_tiers, make_bases
from tests.helpers import tiny_config

pytestmark = pytest.mark.gpu

DEVERR_BAD_TIER, DEVERR_TIER_FULL, DEVERR_BAD_LENGTH = 4, 1, 16


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _cfg8k(**kw):
    return w.get_config(1).with_(**kw)


def _window(cfg, lengths, m=0, integer=False, tail=np.nan, variant_seed=0):
    Ks, Vs = [], []
    for layer in range(m * cfg.layers_per_group, (m + 1) * cfg.layers_per_group):
        K, V = gen_prefill(cfg, layer, lengths=lengths, tail=0.0, variant_seed=variant_seed)
        if integer:
            K = np.clip(np.rint(K.astype(np.float32) * 4), -16, 16).astype(np.float16)
            V = np.clip(np.rint(V.astype(np.float32) * 4), -16, 16).astype(np.float16)
        for X in (K, V):
            for b, n in enumerate(lengths):
                X[b, :, n:] = tail
        Ks.append(K)
        Vs.append(V)
    return Ks, Vs


def _grams(G, cache, cfg, Ks, Vs, lengths, m=0):
    n_dev = G.dev(np.asarray(lengths, np.int32))
    for i, (K, V) in enumerate(zip(Ks, Vs)):
        cache.prefill_gram(m * cfg.layers_per_group + i, G.dev(K), G.dev(V), n_dev, first=(i == 0))
    import torch
    torch.cuda.synchronize()
    return cache.gram(m).cpu().numpy()


def _cache(G, cfg, n):
    return G.make_cache(cfg, n=n, extra=64)


def _oracle_gram(cfg, Ks, Vs, lengths, z, h):
    L = Ks if z == 0 else Vs
    return oracle.window_gram([x for X in L for x in oracle.prefill.window_vectors(X, lengths, h)])


def _abs_gram(cfg, Ks, Vs, lengths, z, h):
    L = Ks if z == 0 else Vs
    return oracle.window_gram([np.abs(x.astype(np.float64)) for X in L
                               for x in oracle.prefill.window_vectors(X, lengths, h)])


@pytest.mark.parametrize("d", [128, 64])
def test_gram_exact_on_integer_data(G, d):
    cfg = _cfg8k(batch=3) if d == 128 else tiny_config(batch=3, num_kv_heads=2, num_q_heads=4, head_dim=64,
                                                        r_max=32, tier_rank=(8, 16, 32), tier_prob=(0.5, 0.3, 0.2),
                                                        n_tokens=3000)
    lengths = [3000, 1777, 0]
    Ks, Vs = _window(cfg, lengths, integer=True)
    cache = _cache(G, cfg, 3000)
    try:
        print(f"gram exact: d={d} lengths={lengths}", flush=True)
        got = _grams(G, cache, cfg, Ks, Vs, lengths)
        for z in range(2):
            for h in range(cfg.num_kv_heads):
                assert np.array_equal(got[z, h], _oracle_gram(cfg, Ks, Vs, lengths, z, h)), (z, h)
        assert cache.check_errors() == 0
        # a second window call sequence starts afresh (first = True)
        got2 = _grams(G, cache, cfg, Ks, Vs, lengths)
        assert np.array_equal(got, got2)
    finally:
        cache.close()


def test_gram_within_fp32_bound_and_ignores_tails(G):
    cfg = _cfg8k(batch=2)
    lengths = [5000, 2345]
    Ks, Vs = _window(cfg, lengths)
    cache = _cache(G, cfg, 5000)
    try:
        got = _grams(G, cache, cfg, Ks, Vs, lengths)
        m = sum(lengths)
        worst = 0.0
        for z in range(2):
            for h in range(cfg.num_kv_heads):
                ref = _oracle_gram(cfg, Ks, Vs, lengths, z, h)
                bound = m * 2.0 ** -24 * _abs_gram(cfg, Ks, Vs, lengths, z, h)
                err = np.abs(got[z, h] - ref)
                assert np.all(np.isfinite(got[z, h]))
                assert np.all(err <= bound), (z, h, (err / np.maximum(bound, 1e-300)).max())
                assert np.array_equal(got[z, h], got[z, h].T)
                worst = max(worst, (err / np.maximum(bound, 1e-300)).max())
        print(f"gram error / bound: {worst:.2e}")
    finally:
        cache.close()


def _ritz_order_gaps(theta):
    th = np.asarray(theta, np.float64)
    gaps = np.full(th.shape, np.inf)
    gaps[:-1] = np.minimum(gaps[:-1], th[:-1] - th[1:])
    gaps[1:] = np.minimum(gaps[1:], th[:-1] - th[1:])
    return gaps


def _bases(G, cache, cfg, omega, q, m=0):
    import torch
    k = omega.shape[-1]
    ritz = torch.zeros((1, 2, cfg.num_kv_heads, k), dtype=torch.float64, device="cuda")
    cache.prefill_bases(m, G.dev(omega[m:m + 1]), q, ritz)
    bk, bv = cache.get_basis(m)
    torch.cuda.synchronize()
    return bk.cpu().numpy(), bv.cpu().numpy(), ritz.cpu().numpy()[0]


@pytest.mark.parametrize("d,k,q", [(128, 72, 2), (128, 72, 0), (64, 40, 1), (64, 64, 3), (64, 41, 2)])
def test_bases_match_oracle_on_identical_gram(G, d, k, q):
    cfg = _cfg8k(batch=2) if d == 128 else tiny_config(batch=2, num_kv_heads=2, num_q_heads=4, head_dim=64,
                                                        r_max=32, tier_rank=(8, 16, 32), tier_prob=(0.5, 0.3, 0.2),
                                                        n_tokens=3000)
    lengths = [3000, 1500]
    Ks, Vs = _window(cfg, lengths, integer=True)
    omega = gen_sketch(cfg, k)
    cache = _cache(G, cfg, 3000)
    try:
        print(f"bases exact-gram: d={d} k={k} q={q}", flush=True)
        _grams(G, cache, cfg, Ks, Vs, lengths)
        bk, bv, ritz = _bases(G, cache, cfg, omega, q)
        ref = oracle.prefill_bases(cfg, Ks, Vs, lengths, omega[0], q)
        strict = 0
        for zi, (z, got) in enumerate((("K", bk), ("V", bv))):
            for h in range(cfg.num_kv_heads):
                th = ref["theta" + z][h]
                assert np.abs(ritz[zi, h] - th).max() <= 1e-10 * th[0], (z, h)
                gaps = _ritz_order_gaps(th)
                B64 = ref[z + "64"][h]
                for i in range(cfg.r_max):
                    if gaps[i] < 1e-6 * th[0]:
                        continue
                    ulp = np.spacing(np.abs(B64[i]).astype(np.float16)).astype(np.float64)
                    diff = np.abs(got[h, i].astype(np.float64) - B64[i])
                    assert np.all(diff <= 0.5 * ulp + 1e-9), (z, h, i, (diff - 0.5 * ulp).max())
                    strict += 1
        assert strict >= cfg.r_max        # most rows are separated
        assert cache.check_errors() == 0
    finally:
        cache.close()


def test_bases_rank_deficient_window(G):
    """A window of 32 vectors per KV head (rank < k = 72): the CholeskyQR
    fast path must decline (a pivot falls to zero) and Gram-Schmidt over
    [Y | I] completes the basis as the oracle does.  Ritz values within
    1e-10 of the largest; every row whose Ritz value is separated (the
    nonzero ones) is the oracle's fp64 row rounded once to fp16."""
    cfg = _cfg8k(batch=2)
    lengths = [5, 3]
    Ks, Vs = _window(cfg, lengths, integer=True)
    omega = gen_sketch(cfg, cfg.r_max + 8)
    cache = _cache(G, cfg, 64)
    try:
        print("bases: rank-deficient window", flush=True)
        _grams(G, cache, cfg, Ks, Vs, lengths)
        bk, bv, ritz = _bases(G, cache, cfg, omega, 2)
        ref = oracle.prefill_bases(cfg, Ks, Vs, lengths, omega[0], 2)
        strict = 0
        for zi, (z, got) in enumerate((("K", bk), ("V", bv))):
            for h in range(cfg.num_kv_heads):
                th = ref["theta" + z][h]
                assert np.abs(ritz[zi, h] - th).max() <= 1e-10 * th[0], (z, h)
                assert (th > 1e-9 * th[0]).sum() <= 32
                gaps = _ritz_order_gaps(th)
                B64 = ref[z + "64"][h]
                for i in range(cfg.r_max):
                    if gaps[i] < 1e-6 * th[0]:
                        continue
                    ulp = np.spacing(np.abs(B64[i]).astype(np.float16)).astype(np.float64)
                    diff = np.abs(got[h, i].astype(np.float64) - B64[i])
                    assert np.all(diff <= 0.5 * ulp + 1e-9), (z, h, i, (diff - 0.5 * ulp).max())
                    strict += 1
        assert strict >= 2 * cfg.num_kv_heads * 16
        assert cache.check_errors() == 0
    finally:
        cache.close()


def test_bases_of_several_windows_in_one_launch(G):
    """One bases call over windows 0..2 (the benchmark's launch shape: every
    window of the model at once), each window with its own Gram sums and
    sketch, against the oracle window by window."""
    import torch
    cfg = _cfg8k(batch=2, num_layers=12)
    lengths = [2000, 1300]
    k, q = cfg.r_max + 8, 2
    omega = gen_sketch(cfg, k)
    cache = _cache(G, cfg, 2000)
    try:
        wins = []
        for m in range(3):
            Ks, Vs = _window(cfg, lengths, m=m, integer=True)
            _grams(G, cache, cfg, Ks, Vs, lengths, m=m)
            wins.append((Ks, Vs))
        ritz = torch.zeros((3, 2, cfg.num_kv_heads, k), dtype=torch.float64, device="cuda")
        cache.prefill_bases(0, G.dev(omega[0:3]), q, ritz)
        torch.cuda.synchronize()
        rz = ritz.cpu().numpy()
        for m, (Ks, Vs) in enumerate(wins):
            bk, bv = (t.cpu().numpy() for t in cache.get_basis(m))
            ref = oracle.prefill_bases(cfg, Ks, Vs, lengths, omega[m], q)
            for zi, (z, got) in enumerate((("K", bk), ("V", bv))):
                for h in range(cfg.num_kv_heads):
                    th = ref["theta" + z][h]
                    assert np.abs(rz[m, zi, h] - th).max() <= 1e-10 * th[0], (m, z, h)
                    gaps = _ritz_order_gaps(th)
                    for i in range(cfg.r_max):
                        if gaps[i] < 1e-6 * th[0]:
                            continue
                        B64 = ref[z + "64"][h][i]
                        ulp = np.spacing(np.abs(B64).astype(np.float16)).astype(np.float64)
                        assert np.all(np.abs(got[h, i].astype(np.float64) - B64) <= 0.5 * ulp + 1e-9), (m, z, h, i)
        assert cache.check_errors() == 0
    finally:
        cache.close()


def test_bases_match_oracle_on_gaussian_data(G):
    cfg = _cfg8k(batch=2)
    lengths = [4000, 2100]
    Ks, Vs = _window(cfg, lengths)
    k, q = cfg.r_max + 8, 2
    omega = gen_sketch(cfg, k)
    cache = _cache(G, cfg, 4000)
    try:
        grams = _grams(G, cache, cfg, Ks, Vs, lengths)
        bk, bv, ritz = _bases(G, cache, cfg, omega, q)
        ref = oracle.prefill_bases(cfg, Ks, Vs, lengths, omega[0], q)
        for zi, (z, got) in enumerate((("K", bk), ("V", bv))):
            for h in range(cfg.num_kv_heads):
                C = ref["gram" + z][h]
                dC = np.linalg.norm(grams[zi, h] - C, 2)
                th = ref["theta" + z][h]
                assert np.abs(ritz[zi, h] - th).max() <= 2 * dC + 1e-10 * th[0], (z, h)
                gaps = _ritz_order_gaps(th)
                B64 = ref[z + "64"][h]
                for i in range(cfg.r_max):
                    v = B64[i]
                    res = np.linalg.norm(C @ v - th[i] * v) / th[0]
                    if res > 1e-9 or gaps[i] < 100 * dC:
                        continue
                    ulp = np.spacing(np.abs(v).astype(np.float16)).astype(np.float64)
                    tol = 0.5 * ulp + 2 * np.sqrt(2) * dC / gaps[i] + 1e-9
                    assert np.all(np.abs(got[h, i].astype(np.float64) - v) <= tol), (z, h, i)
    finally:
        cache.close()


def _encode(G, cache, cfg, layer, K, V, lengths, tier, gK=None, gV=None):
    cache.prefill_encode(layer, G.dev(K), G.dev(V), G.dev(np.asarray(lengths, np.int32)), G.dev(tier),
                         None if gK is None else G.dev(gK), None if gV is None else G.dev(gV))


def _compare_layer(cfg, got, ref, lengths):
    cb = cfg.coef_bits
    fields = ["tier"] + [f + z for z in "KV" for f in ("coef", "idx", "val", "scale")]
    if cb == 8:
        fields += ["cscaleK", "cscaleV"]
    for b, n in enumerate(lengths):
        for f in fields:
            g = got[f][b, :, :n]
            r = ref[f][b, :, :n]
            if f.startswith(("idx", "val")):
                # only each token's own s_k entries are defined
                res = np.asarray(cfg.resid_per_tier)[ref["tier"][b, :, :n]]
                mask = np.arange(cfg.s_max)[None, None, :] < res[..., None]
                g, r = np.where(mask, g[..., :cfg.s_max], 0), np.where(mask, r, 0)
            if f.startswith("scale"):
                res = np.asarray(cfg.resid_per_tier)[ref["tier"][b, :, :n]]
                g, r = np.where(res > 0, g.view(np.uint16), 0), np.where(res > 0, r.view(np.uint16), 0)
            gv = g.view(np.uint16) if g.dtype == np.float16 else g
            rv = r.view(np.uint16) if r.dtype == np.float16 else r
            bad = np.argwhere(gv != rv)
            assert bad.size == 0, f"b={b} {f}: {len(bad)} mismatches, first {bad[:3].tolist()}"


CASES = {
    "fp16": dict(cfg=lambda: _cfg8k(batch=3), gates=True),
    "int8coef": dict(cfg=lambda: _cfg8k(batch=3, coef_bits=8), gates=True),
    "d64_8bit_resid": dict(cfg=lambda: tiny_config(batch=3, num_kv_heads=2, num_q_heads=8, head_dim=64, r_max=32,
                                                   tier_rank=(4, 8, 16, 32), tier_prob=(0.4, 0.3, 0.2, 0.1),
                                                   resid_channels=4, resid_bits=8, n_tokens=3000), gates=False),
    "paper_literal": dict(cfg=lambda: _cfg8k(batch=3, r_max=32, tier_rank=(32,) * 4, tier_prob=(0.4, 0.3, 0.2, 0.1),
                                             tier_resid=(0, 2, 4, 8)), gates=True),
    # ranks 4 mod 8: the encoder's 4-row remainder block in both steps, with
    # 8-bit and fp16 coefficients
    "ranks_4mod8_int8coef": dict(cfg=lambda: _cfg8k(batch=3, r_max=44, tier_rank=(4, 12, 20, 44),
                                                    tier_prob=(0.4, 0.3, 0.2, 0.1), coef_bits=8), gates=True),
    "ranks_4mod8_fp16": dict(cfg=lambda: _cfg8k(batch=3, r_max=44, tier_rank=(4, 12, 20, 44),
                                                tier_prob=(0.4, 0.3, 0.2, 0.1)), gates=False),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_prefill_encode_bit_exact(G, case):
    cfg = CASES[case]["cfg"]()
    lengths = [3000, 1777, 0]
    layer = cfg.layers_per_group + 1 if cfg.num_layers > cfg.layers_per_group else 0
    m = layer // cfg.layers_per_group
    bases = make_bases(cfg)
    K, V = gen_prefill(cfg, layer, lengths=lengths, tail=np.nan)
    tier = gen_tiers(cfg, layer, 3000)
    gK, gV = gen_gates(cfg, layer, 3000) if CASES[case]["gates"] else (None, None)
    cache = _cache(G, cfg, 3000)
    try:
        G.load_bases(cache, bases, groups=[m])
        print(f"prefill encode: {case} lengths={lengths}", flush=True)
        _encode(G, cache, cfg, layer, K, V, lengths, tier, gK, gV)
        assert cache.check_errors() == 0
        got, counts, _ = G.export_np(cache, layer, cfg.batch, 3000)
        ref = oracle.prefill_encode(cfg, bases["K"][m], bases["V"][m], K, V, lengths, tier, gK, gV)
        _compare_layer(cfg, got, ref, lengths)
        for b, n in enumerate(lengths):
            for h in range(cfg.num_kv_heads):
                assert list(counts[b, h]) == [int((tier[b, h, :n] == k).sum()) for k in range(cfg.num_tiers)]
    finally:
        cache.close()


def test_prefill_batch16_ragged(G):
    """Sixteen sequences of different lengths (the batch of the 32K x 16
    workload, shorter), including empty ones: Gram sums exact on integer
    data, bases and the bulk encode against the oracle."""
    cfg = _cfg8k(batch=16)
    rng = np.random.default_rng(16)
    lengths = [int(x) for x in rng.integers(0, 1200, 16)]
    lengths[3] = 0
    lengths[7] = 1199
    n = max(lengths)
    Ks, Vs = _window(cfg, lengths, integer=True)
    omega = gen_sketch(cfg, cfg.r_max + 8)
    cache = _cache(G, cfg, n)
    try:
        got = _grams(G, cache, cfg, Ks, Vs, lengths)
        for z in range(2):
            for h in range(cfg.num_kv_heads):
                assert np.array_equal(got[z, h], _oracle_gram(cfg, Ks, Vs, lengths, z, h)), (z, h)
        bk, bv, ritz = _bases(G, cache, cfg, omega, 2)
        ref = oracle.prefill_bases(cfg, Ks, Vs, lengths, omega[0], 2)
        for zi, z in enumerate("KV"):
            for h in range(cfg.num_kv_heads):
                th = ref["theta" + z][h]
                assert np.abs(ritz[zi, h] - th).max() <= 1e-10 * th[0], (z, h)
        layer = 2
        tier = gen_tiers(cfg, layer, n)
        bases = {"K": ref["K"][None], "V": ref["V"][None]}
        G.load_bases(cache, bases, groups=[0])
        _encode(G, cache, cfg, layer, Ks[layer], Vs[layer], lengths, tier)
        assert cache.check_errors() == 0
        out, _, _ = G.export_np(cache, layer, cfg.batch, n)
        ref_lay = oracle.prefill_encode(cfg, ref["K"], ref["V"], Ks[layer], Vs[layer], lengths, tier)
        _compare_layer(cfg, out, ref_lay, lengths)
    finally:
        cache.close()


def _permutation_bases(cfg, seed):
    """Signed permutation rows (fp16-exact): every coefficient is a signed
    input channel and every residual channel is an input value or exactly 0."""
    rng = np.random.default_rng(seed)
    out = {}
    for z in "KV":
        B = np.zeros((cfg.num_groups, cfg.num_kv_heads, cfg.r_max, cfg.head_dim), np.float16)
        for m in range(cfg.num_groups):
            for h in range(cfg.num_kv_heads):
                cols = rng.permutation(cfg.head_dim)[: cfg.r_max]
                B[m, h, np.arange(cfg.r_max), cols] = rng.choice([-1.0, 1.0], cfg.r_max)
        out[z] = B
    return out


@pytest.mark.parametrize("coef_bits", [16, 8])
def test_prefill_encode_planted_ties(G, coef_bits):
    """Residuals with many equal |e| at the kept-channel threshold (values
    from {0, +-0.25, +-0.5, +-1}) and all-zero residuals, after a run of
    generic tokens, in one call: the tie rule (the lower channel first) and
    the tie-free channel selection against the oracle, bit-exact."""
    cfg = _cfg8k(batch=2, coef_bits=coef_bits)
    lengths = [2400, 1500]
    n = max(lengths)
    layer = 1
    bases = _permutation_bases(cfg, 7)
    K, V = gen_prefill(cfg, layer, lengths=lengths, tail=np.nan)
    rng = np.random.default_rng(11)
    for X in (K, V):
        planted = rng.choice([0.0, 0.25, -0.25, 0.5, -0.5, 1.0, -1.0], (cfg.batch, cfg.num_kv_heads, n, cfg.head_dim))
        X[:, :, 800:n] = planted[:, :, 800:n].astype(np.float16)
        X[:, :, 1200:1300] = 0.0
        for b, nb in enumerate(lengths):
            X[b, :, nb:] = np.nan
    tier = gen_tiers(cfg, layer, n)
    cache = _cache(G, cfg, n)
    try:
        G.load_bases(cache, bases, groups=[0])
        print(f"prefill encode with planted ties: coef_bits={coef_bits}", flush=True)
        _encode(G, cache, cfg, layer, K, V, lengths, tier)
        assert cache.check_errors() == 0
        got, _, _ = G.export_np(cache, layer, cfg.batch, n)
        ref = oracle.prefill_encode(cfg, bases["K"][0], bases["V"][0], K, V, lengths, tier)
        _compare_layer(cfg, got, ref, lengths)
        # the all-zero rows have a zero scale, and (fp16 coefficients: each
        # residual channel is the input channel or 0) the planted rows put
        # more channels at the threshold than are kept
        assert (ref["scaleK"][0, :, 1200:1300].view(np.uint16) == 0).all()
        if coef_bits == 16:
            s = cfg.resid_per_tier[0]
            B = bases["K"][0, 0].astype(np.float64)
            x = K[0, 0, 800:1200].astype(np.float64)
            e = np.abs(x - (x @ B.T) @ B)
            top = -np.sort(-e, axis=1)
            assert (top[:, s] == top[:, s - 1]).sum() > 100
    finally:
        cache.close()


def test_prefill_encode_in_two_chunks_equals_one(G):
    """1000 positions, then the remaining 2000 in a second call: the layer is
    the oracle's encoding of all 3000 (positions continue)."""
    cfg = _cfg8k(batch=2)
    layer, n, cut = 2, 3000, 1000
    bases = make_bases(cfg)
    K, V = gen_prefill(cfg, layer, lengths=[n, n])
    tier = gen_tiers(cfg, layer, n)
    gK, gV = gen_gates(cfg, layer, n)
    cache = _cache(G, cfg, n)
    try:
        G.load_bases(cache, bases, groups=[0])
        _encode(G, cache, cfg, layer, K[:, :, :cut].copy(), V[:, :, :cut].copy(), [cut, cut],
                tier[:, :, :cut].copy(), gK[:, :, :cut].copy(), gV[:, :, :cut].copy())
        _encode(G, cache, cfg, layer, K[:, :, cut:].copy(), V[:, :, cut:].copy(), [n - cut, n - cut],
                tier[:, :, cut:].copy(), gK[:, :, cut:].copy(), gV[:, :, cut:].copy())
        assert cache.check_errors() == 0
        got, _, _ = G.export_np(cache, layer, cfg.batch, n)
        ref = oracle.prefill_encode(cfg, bases["K"][0], bases["V"][0], K, V, [n, n], tier, gK, gV)
        _compare_layer(cfg, got, ref, [n, n])
    finally:
        cache.close()


def test_prefill_encode_refusals(G):
    """A tier beyond the table refuses its (sequence, KV head) as a whole;
    the others are encoded.  A tier region that would overflow does the
    same."""
    cfg = _cfg8k(batch=2)
    layer, n = 0, 1000
    bases = make_bases(cfg)
    K, V = gen_prefill(cfg, layer, lengths=[n, n])
    tier = gen_tiers(cfg, layer, n)
    tier[1, 3, 500] = cfg.num_tiers            # one bad token
    cache = _cache(G, cfg, n)
    try:
        G.load_bases(cache, bases, groups=[0])
        _encode(G, cache, cfg, layer, K, V, [n, n], tier)
        assert cache.check_errors() & DEVERR_BAD_TIER
        counts = cache.read_counts(layer, cfg.batch)
        assert counts[1, 3].sum() == 0
        assert counts[0].sum() == cfg.num_kv_heads * n and counts[1].sum() == (cfg.num_kv_heads - 1) * n
        cache.clear_errors()
        got, _, _ = G.export_np(cache, layer, cfg.batch, n)
        ref = oracle.prefill_encode(cfg, bases["K"][0], bases["V"][0], K[:1], V[:1], [n], tier[:1])
        for f in ("coefK", "scaleV", "idxK"):
            assert np.array_equal(got[f][0].view(np.uint8), ref[f][0].view(np.uint8))
    finally:
        cache.close()
    # a tier region too small for the prefill
    small = G.make_cache(cfg, capacity=[n // 4, n, n, n], max_tokens=n + 16, n=n)
    try:
        G.load_bases(small, bases, groups=[0])
        tier = gen_tiers(cfg, layer, n)
        _encode(G, small, cfg, layer, K, V, [n, n], tier)
        assert small.check_errors() & DEVERR_TIER_FULL
        assert small.read_counts(layer, cfg.batch).sum() == 0
    finally:
        small.close()


def test_appends_after_prefill_continue_the_layer(G):
    """Prefill encode, then three one-token appends (dwkv_append) and one
    one-launch decode step: the position map and tier slots the prefill
    leaves are the ones the append path continues; the exported layer is the
    oracle's prefill encoding followed by the oracle's appends."""
    import torch
    cfg = _cfg8k(batch=2)
    layer, lengths = 3, [900, 555]
    bases = make_bases(cfg)
    K, V = gen_prefill(cfg, layer, lengths=lengths)
    tier = gen_tiers(cfg, layer, 900)
    gK, gV = gen_gates(cfg, layer, 900)
    cache = _cache(G, cfg, 1000)
    try:
        G.load_bases(cache, bases, groups=[0])
        _encode(G, cache, cfg, layer, K, V, lengths, tier, gK, gV)
        apps = [w.gen_append_inputs(cfg, layer, st, bases) for st in range(4)]
        for a in apps[:3]:
            cache.append(layer, G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"]))
        q = gen_query(cfg, layer)
        cache.decode_step(layer, G.dev(q), G.dev(apps[3]["k"]), G.dev(apps[3]["v"]), G.dev(apps[3]["tier"]))
        torch.cuda.synchronize()
        assert cache.check_errors() == 0
        n_after = [n + 4 for n in lengths]
        got, counts, _ = G.export_np(cache, layer, cfg.batch, max(n_after))
        ref = oracle.prefill_encode(cfg, bases["K"][0], bases["V"][0], K, V, lengths, tier, gK, gV)
        for b, n in enumerate(lengths):
            for h in range(cfg.num_kv_heads):
                for st, a in enumerate(apps):
                    t = n + st
                    k = int(a["tier"][b, h])
                    assert got["tier"][b, h, t] == k
                    r, s_ = cfg.tier_rank[k], cfg.resid_per_tier[k]
                    for z in "KV":
                        enc = oracle.append_vector(bases[z][0][h], a[z.lower()][b, h], r, s_, cfg.qmax)
                        assert np.array_equal(got["coef" + z][b, h, t, :r].view(np.uint16), enc[0].view(np.uint16))
                        assert np.array_equal(got["idx" + z][b, h, t, :s_], enc[1])
                        assert np.array_equal(got["val" + z][b, h, t, :s_], enc[2])
                        assert got["scale" + z][b, h, t].view(np.uint16) == enc[3].view(np.uint16)
        _compare_layer(cfg, {kk: np.ascontiguousarray(v[:, :, :900]) for kk, v in got.items()}, ref, lengths)
    finally:
        cache.close()


def test_prefill_pipelined_on_two_streams(G):
    """Each window's bases on a second stream as soon as its Gram sums are
    complete, overlapping the next windows' Gram sums, and each window's
    encodes waiting for its bases only, all on one workspace: the bases and
    every encoded layer equal those of the sequential order, bit for bit."""
    import torch
    cfg = _cfg8k(batch=2)
    lengths, n, nw = [1500, 900], 1500, 3
    lpg = cfg.layers_per_group
    layers = range(nw * lpg)
    data = {l: gen_prefill(cfg, l, lengths=lengths, tail=0.0) for l in layers}
    tiers = {l: G.dev(gen_tiers(cfg, l, n)) for l in layers}
    dev = {l: (G.dev(data[l][0]), G.dev(data[l][1])) for l in layers}
    omega = G.dev(gen_sketch(cfg, cfg.r_max + 8)[:nw])
    nd = G.dev(np.asarray(lengths, np.int32))
    seq, pipe = _cache(G, cfg, n), _cache(G, cfg, n)
    try:
        print("prefill: sequential order", flush=True)
        for l in layers:
            seq.prefill_gram(l, *dev[l], nd, first=(l % lpg == 0))
        seq.prefill_bases(0, omega, 2)
        for l in layers:
            seq.prefill_encode(l, *dev[l], nd, tiers[l])
        torch.cuda.synchronize()
        print("prefill: pipelined on two streams", flush=True)
        main, side = torch.cuda.current_stream(), torch.cuda.Stream()
        ev_gram = [torch.cuda.Event() for _ in range(nw)]
        ev_bases = [torch.cuda.Event() for _ in range(nw)]
        for m in range(nw):
            for l in range(m * lpg, (m + 1) * lpg):
                pipe.prefill_gram(l, *dev[l], nd, first=(l % lpg == 0))
            ev_gram[m].record(main)
            with torch.cuda.stream(side):
                side.wait_event(ev_gram[m])
                pipe.prefill_bases(m, omega[m:m + 1], 2)
                ev_bases[m].record(side)
        for m in range(nw):
            main.wait_event(ev_bases[m])
            for l in range(m * lpg, (m + 1) * lpg):
                pipe.prefill_encode(l, *dev[l], nd, tiers[l])
        torch.cuda.synchronize()
        assert seq.check_errors() == 0 and pipe.check_errors() == 0
        for m in range(nw):
            for a, b in zip(seq.get_basis(m), pipe.get_basis(m)):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), m
        for l in layers:
            ga, ca, _ = G.export_np(seq, l, cfg.batch, n)
            gb, cb, _ = G.export_np(pipe, l, cfg.batch, n)
            assert np.array_equal(ca, cb), l
            for f in ga:
                assert np.array_equal(ga[f].view(np.uint8), gb[f].view(np.uint8)), (l, f)
    finally:
        seq.close()
        pipe.close()


def test_prefill_encode_follows_new_bases(G):
    """The encoder's copy of a window's bases is reused by the next layers of
    that window and remade after dwkv_set_basis: layer 0 with bases A, layer
    1 with A again, then layer 2 after the window's bases become B; each
    against the oracle with the bases it was encoded with."""
    cfg = _cfg8k(batch=2)
    lengths, n = [700, 450], 700
    A, B = make_bases(cfg), make_bases(cfg, variant_seed=1)
    cache = _cache(G, cfg, n)
    try:
        for layer, bases in ((0, A), (1, A), (2, B)):
            if layer != 1:
                G.load_bases(cache, bases, groups=[0])
            K, V = gen_prefill(cfg, layer, lengths=lengths)
            tier = gen_tiers(cfg, layer, n)
            print(f"prefill encode after bases change: layer {layer}", flush=True)
            _encode(G, cache, cfg, layer, K, V, lengths, tier)
            assert cache.check_errors() == 0
            got, _, _ = G.export_np(cache, layer, cfg.batch, n)
            ref = oracle.prefill_encode(cfg, bases["K"][0], bases["V"][0], K, V, lengths, tier)
            _compare_layer(cfg, got, ref, lengths)
    finally:
        cache.close()


def test_prefill_basis_copy_shared_workspace_and_graphs(G):
    """The encoder's block copy of a window's bases lives in the workspace:
    (1) two caches sharing one workspace each encode with their own bases;
    (2) an encode captured in a graph makes its own copy, so replaying the
    graph after another window's encode overwrote the copy still uses the
    right bases.  Every layer against the oracle with its bases."""
    import torch
    from compressed_kv_cache_dwkv_amd import dwkv_prefill_encode
    cfg = _cfg8k(batch=2)
    lengths, n = [500, 320], 500
    lpg = cfg.layers_per_group
    A, B = make_bases(cfg), make_bases(cfg, variant_seed=1)
    ca, cb = _cache(G, cfg, n), _cache(G, cfg, n)
    nd = G.dev(np.asarray(lengths, np.int32))
    inputs = {}

    def prepare(cache, layer):
        K, V = gen_prefill(cfg, layer, lengths=lengths)
        tier = gen_tiers(cfg, layer, n)
        inputs[(id(cache), layer)] = (K, V, tier, G.dev(K), G.dev(V), G.dev(tier))

    def enc(cache, layer, ws):
        if (id(cache), layer) not in inputs:
            prepare(cache, layer)
        dk, dv, dt = inputs[(id(cache), layer)][3:]
        dwkv_prefill_encode(cache.handle, layer, dk, dv, nd, dt, ws)

    def check(cache, layer, bases, m):
        K, V, tier = inputs[(id(cache), layer)][:3]
        got, _, _ = G.export_np(cache, layer, cfg.batch, n)
        ref = oracle.prefill_encode(cfg, bases["K"][m], bases["V"][m], K, V, lengths, tier)
        _compare_layer(cfg, got, ref, lengths)

    try:
        ws = ca.prefill_workspace()
        G.load_bases(ca, A, groups=[0, 1])
        G.load_bases(cb, B, groups=[0])
        print("shared workspace: cache A, cache B, cache A", flush=True)
        enc(ca, 0, ws)
        enc(cb, 0, ws)
        enc(ca, 1, ws)
        torch.cuda.synchronize()
        assert ca.check_errors() == 0 and cb.check_errors() == 0
        check(ca, 0, A, 0)
        check(cb, 0, B, 0)
        check(ca, 1, A, 0)
        print("graph: capture an encode of window 0, then an eager encode of window 1, then replay", flush=True)
        enc(ca, 2, ws)                       # eager copy of window 0's bases
        prepare(ca, 3)                       # (no uploads inside the capture)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            enc(ca, 3, ws)                   # window 0 again, inside the capture
        enc(ca, lpg, ws)                     # window 1: its copy replaces window 0's
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert ca.check_errors() == 0
        check(ca, 2, A, 0)
        check(ca, 3, A, 0)
        check(ca, lpg, A, 1)
    finally:
        ca.close()
        cb.close()


def test_prefill_length_beyond_the_buffer_is_refused(G):
    """n_tokens > n_cap sets the bad-length bit and leaves that sequence's
    heads empty; the other sequence is encoded."""
    cfg = _cfg8k(batch=2)
    layer = 1
    bases = make_bases(cfg)
    K, V = gen_prefill(cfg, layer, lengths=[300, 300])
    tier = gen_tiers(cfg, layer, 300)
    cache = _cache(G, cfg, 1000)
    try:
        G.load_bases(cache, bases, groups=[0])
        cache.prefill_encode(layer, G.dev(K), G.dev(V), G.dev(np.asarray([300, 301], np.int32)), G.dev(tier))
        assert cache.check_errors() & DEVERR_BAD_LENGTH
        counts = cache.read_counts(layer, cfg.batch)
        assert counts[1].sum() == 0 and counts[0].sum() == cfg.num_kv_heads * 300
    finally:
        cache.close()


def test_prefill_chain_decodes_like_the_oracle_chain(G):
    """Gram, bases and encode for a window, then decode attention: the GPU
    chain's error against dense attention over the original keys and
    values is that of the oracle's own chain."""
    import torch
    cfg = _cfg8k(batch=2)
    lengths = [4000, 2500]
    Ks, Vs = _window(cfg, lengths, tail=0.0)
    k, q = cfg.r_max + 8, 2
    omega = gen_sketch(cfg, k)
    cache = _cache(G, cfg, 4000)
    try:
        _grams(G, cache, cfg, Ks, Vs, lengths)
        cache.prefill_bases(0, G.dev(omega[0:1]), q)
        for i in range(cfg.layers_per_group):
            tier = gen_tiers(cfg, i, 4000)
            _encode(G, cache, cfg, i, Ks[i], Vs[i], lengths, tier)
        assert cache.check_errors() == 0
        ref = oracle.prefill_bases(cfg, Ks, Vs, lengths, omega[0], q)
        for i in (0, cfg.layers_per_group - 1):
            qv = gen_query(cfg, i)
            got = G.decode_np(cache, i, qv)
            dense = oracle.dense_decode(Ks[i], Vs[i], lengths, qv)
            lay = oracle.prefill_encode(cfg, ref["K"], ref["V"], Ks[i], Vs[i], lengths, gen_tiers(cfg, i, 4000))
            chain = oracle.decode(cfg, lay, ref["K"], ref["V"], qv)
            e_gpu = G.norm_err(got, dense).max()
            e_or = G.norm_err(chain, dense).max()
            print(f"layer {i}: gpu chain {e_gpu:.3e}, oracle chain {e_or:.3e}")
            assert e_gpu <= 1.5 * e_or + 2e-3
    finally:
        cache.close()


def test_prefill_full_size_64k(G):
    """The 64K-token Llama-3-8B shape of the benchmark (one window: 4
    layers, 8 KV heads): the Gram sums within the fp32 bound, the Ritz
    values within Weyl's bound, and 4096 sampled tokens of each layer
    encoded bit-exactly."""
    import torch
    cfg = w.get_config(2)
    n = cfg.n_tokens
    lengths = [n]
    print("prefill 64K: generating", flush=True)
    Ks, Vs = _window(cfg, lengths, tail=0.0)
    k, q = cfg.r_max + 8, 2
    omega = gen_sketch(cfg, k)
    cache = _cache(G, cfg, n)
    try:
        print("prefill 64K: gram", flush=True)
        grams = _grams(G, cache, cfg, Ks, Vs, lengths)
        bk, bv, ritz = _bases(G, cache, cfg, omega, q)
        tiers = [gen_tiers(cfg, i, n) for i in range(cfg.layers_per_group)]
        for i in range(cfg.layers_per_group):
            _encode(G, cache, cfg, i, Ks[i], Vs[i], lengths, tiers[i])
        assert cache.check_errors() == 0
        print("prefill 64K: oracle", flush=True)
        ref = oracle.prefill_bases(cfg, Ks, Vs, lengths, omega[0], q)
        for zi, z in enumerate("KV"):
            for h in range(cfg.num_kv_heads):
                C = ref["gram" + z][h]
                bound = n * cfg.layers_per_group * 2.0 ** -24 * _abs_gram(cfg, Ks, Vs, lengths, zi, h)
                assert np.all(np.abs(grams[zi, h] - C) <= bound)
                dC = np.linalg.norm(grams[zi, h] - C, 2)
                th = ref["theta" + z][h]
                assert np.abs(ritz[zi, h] - th).max() <= 2 * dC + 1e-10 * th[0]
        # the encoder at this shape, on the oracle's bases (an oracle input
        # never comes from the GPU), against the oracle on a token sample
        bases = {"K": ref["K"][None], "V": ref["V"][None]}
        rng = np.random.default_rng(7)
        sample = np.sort(rng.choice(n, 4096, replace=False))
        for i in (0, cfg.layers_per_group - 1):
            fresh = _cache(G, cfg, n)
            try:
                G.load_bases(fresh, bases, groups=[0])
                _encode(G, fresh, cfg, i, Ks[i], Vs[i], lengths, tiers[i])
                assert fresh.check_errors() == 0
                got, _, _ = G.export_np(fresh, i, 1, n)
            finally:
                fresh.close()
            sub = {k2: np.ascontiguousarray(v[:, :, sample]) for k2, v in got.items()}
            ref_lay = oracle.prefill_encode(cfg, ref["K"], ref["V"], np.ascontiguousarray(Ks[i][:, :, sample]),
                                            np.ascontiguousarray(Vs[i][:, :, sample]), [len(sample)],
                                            np.ascontiguousarray(tiers[i][:, :, sample]))
            _compare_layer(cfg, sub, ref_lay, [len(sample)])
    finally:
        cache.close()
