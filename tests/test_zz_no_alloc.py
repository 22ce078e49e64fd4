"""dwkv_decode_step_noalloc -- the one-launch decode step with the library's
static scratch array in place of a caller workspace -- against
dwkv_decode_step, the entry point it is a variant of (needs an MI355X).

Both run the same kernel with the same split count, so the output must be
bitwise identical and the cache after the step byte for byte the same; the
output also meets the oracle's 2e-3 row-max-normalised bound and the
appended token the oracle's encoding bit for bit.  Two calls in a row on
two caches: first the larger input (the 70B shape, 8 query heads per KV
head, 32 splits), then a smaller one (the 8B shape, two sequences, fewer
splits) whose counters and partials land where the first call's partials
were."""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases
from tests.test_append_gpu import _compare_token

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _one_call(G, cfg, n0, layer, splits, ragged=None):
    import torch
    import compressed_kv_cache_dwkv_amd as d
    bases = make_bases(cfg)
    m = layer // cfg.layers_per_group
    caches = [G.make_cache(cfg, n=n0, extra=4, splits=splits) for _ in range(2)]
    ref_cache, na_cache = caches
    try:
        print(f"no-alloc test: {cfg.name} batch={cfg.batch} n0={n0} layer={layer} "
              f"splits={na_cache.splits}", flush=True)
        lay = gen_layer(cfg, layer, n=n0)
        if ragged is not None:
            lay["n_tokens"][:] = ragged
        for c in caches:
            G.load_bases(c, bases, groups=[m])
            G.load_layer(c, layer, lay)
        q = gen_query(cfg, layer, step=1)
        a = gen_append_inputs(cfg, layer, 1, bases)
        before = na_cache.read_counts(layer, cfg.batch)
        dq, dk, dv, dt = G.dev(q), G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"])
        out_ref = ref_cache.decode_step(layer, dq, dk, dv, dt)
        out_na = torch.empty_like(out_ref)
        d.dwkv_decode_step_noalloc(na_cache.handle, layer, dq, out_na, dk, dv, dt)
        torch.cuda.synchronize()
        got, want = out_na.cpu().numpy(), out_ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "output differs from dwkv_decode_step"
        ref = oracle.decode(cfg, lay, bases["K"][m], bases["V"][m], q)
        err = G.norm_err(got.astype(np.float64), ref)
        if ragged is not None:
            err = err[np.asarray(ragged) > 0]
        assert err.max() <= TOL, f"max normalised error {err.max():.3e}"
        n_max = int(lay["n_tokens"].max()) + 1
        ex_r, cnt_r, sl_r = G.export_np(ref_cache, layer, cfg.batch, n_max)
        ex_n, cnt_n, sl_n = G.export_np(na_cache, layer, cfg.batch, n_max)
        assert np.array_equal(cnt_r, cnt_n) and np.array_equal(sl_r, sl_n)
        for key in ex_r:
            assert np.array_equal(ex_r[key].view(np.uint8), ex_n[key].view(np.uint8)), key
        enc = oracle.append_layer(cfg, bases["K"][m], bases["V"][m], a["k"], a["v"], a["tier"])
        for b in range(cfg.batch):
            pos = int(lay["n_tokens"][b])
            sub = {k: v[b:b + 1] for k, v in ex_n.items()}
            _compare_token(cfg.with_(batch=1), sub, sl_n[b:b + 1], before[b:b + 1], pos,
                           {k: v[b:b + 1] for k, v in enc.items()}, a["tier"][b:b + 1])
        for c in caches:
            assert c.check_errors() == 0
    finally:
        for c in caches:
            c.close()


def test_noalloc_step_matches_workspace_step_on_two_calls(G):
    _one_call(G, w.get_config(4), 20000, layer=9, splits=32)
    _one_call(G, w.get_config(1).with_(batch=2), 1500, layer=6, splits=4, ragged=[1500, 700])


def test_noalloc_step_replayed_from_a_graph(G):
    """The callers this entry point is for capture it in graphs.  One eager
    call sets the scratch up, then the captured call is replayed for three
    more steps, each step's query and token written into the graph's input
    buffers between replays: every replay's output bitwise equal to
    dwkv_decode_step's on a twin cache, and the layers byte for byte the
    same at the end (the split merge leaves the scratch's counters at zero
    for the next replay)."""
    import torch
    import compressed_kv_cache_dwkv_amd as d
    cfg = w.get_config(1)
    layer, n0, steps = 5, 8192, 4
    bases = make_bases(cfg)
    m = layer // cfg.layers_per_group
    caches = [G.make_cache(cfg, n=n0, extra=steps + 4, splits=32) for _ in range(2)]
    ref_cache, na_cache = caches
    try:
        print(f"no-alloc graph test: {cfg.name} n0={n0} layer={layer} splits={na_cache.splits}", flush=True)
        lay = gen_layer(cfg, layer, n=n0)
        for c in caches:
            G.load_bases(c, bases, groups=[m])
            G.load_layer(c, layer, lay)
        B, Hq, Hkv, dh = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
        sq = torch.zeros((B, Hq, dh), dtype=torch.float16, device="cuda")
        sk = torch.zeros((B, Hkv, dh), dtype=torch.float16, device="cuda")
        sv = torch.zeros_like(sk)
        st = torch.zeros((B, Hkv), dtype=torch.uint8, device="cuda")
        so = torch.zeros((B, Hq, dh), dtype=torch.float32, device="cuda")
        g = None
        for step in range(steps):
            q = gen_query(cfg, layer, step=step)
            a = gen_append_inputs(cfg, layer, step, bases)
            want = ref_cache.decode_step(layer, G.dev(q), G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"]))
            sq.copy_(G.dev(q))
            sk.copy_(G.dev(a["k"]))
            sv.copy_(G.dev(a["v"]))
            st.copy_(G.dev(a["tier"]))
            if g is None:       # the first call is eager; the graph is captured after it
                d.dwkv_decode_step_noalloc(na_cache.handle, layer, sq, so, sk, sv, st)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    d.dwkv_decode_step_noalloc(na_cache.handle, layer, sq, so, sk, sv, st)
            else:
                g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(so.cpu().numpy().view(np.uint32), want.cpu().numpy().view(np.uint32)), \
                f"step {step}: differs from dwkv_decode_step"
            if step == 0:
                ref = oracle.decode(cfg, lay, bases["K"][m], bases["V"][m], q)
                err = G.norm_err(so.cpu().numpy().astype(np.float64), ref)
                assert err.max() <= TOL, f"max normalised error {err.max():.3e}"
            print(f"  step {step}: {'eager' if step == 0 else 'replay'} equal to dwkv_decode_step", flush=True)
        ex_r, cnt_r, sl_r = G.export_np(ref_cache, layer, B, n0 + steps)
        ex_n, cnt_n, sl_n = G.export_np(na_cache, layer, B, n0 + steps)
        assert np.array_equal(cnt_r, cnt_n) and np.array_equal(sl_r, sl_n)
        assert int(cnt_n.sum()) == B * Hkv * (n0 + steps)
        for key in ex_r:
            assert np.array_equal(ex_r[key].view(np.uint8), ex_n[key].view(np.uint8)), key
        for c in caches:
            assert c.check_errors() == 0
        del g
    finally:
        for c in caches:
            c.close()
