"""The one-launch decode step and the decode attention replayed from HIP
graphs, as the benchmark launches them, against the same calls launched
eagerly (needs an MI355X).

A graph records its launches with their arguments fixed, so every replay
reads its inputs from the same buffers and writes the same output buffers.
Between replays the test writes the next step's query and new token into
those buffers and runs eager work of its own on the graph's cache (a decode
through the same workspace), synchronises, and compares.  Two caches start
from the same layers: one steps eagerly, the other by replays.  The same
kernel with the same split count over the same data is deterministic, so
each replay's outputs must equal the eager step's bit for bit, and the
layers must end byte for byte the same (counts, slots and every stored
field).  The arrival counters that the split merge uses are left at zero by
each launch, so no clear is recorded in the graph.  The first step's output
is also checked against the oracle (2e-3 row-max normalised)."""
import numpy as np
import pytest

import oracle
import workload as w
from workload.gen import gen_append_inputs, gen_layer, gen_query, make_bases

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def G():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_util
    return gpu_util


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("ci,n0,layers,splits,steps", [
    (1, 8192, (5, 6), 32, 3),      # Llama-3-8B shape, the benchmark's 32 splits, two layers per replay
    (4, 3000, (9,), 32, 2),        # Llama-3-70B shape: 8 query heads per KV head
    (3, 1200, (2,), 3, 2),         # 16 sequences, few splits per head
])
def test_step_graph_replays_equal_eager_steps(G, ci, n0, layers, splits, steps):
    import torch
    cfg = w.get_config(ci)
    bases = make_bases(cfg)
    groups = sorted({l // cfg.layers_per_group for l in layers})
    caches = [G.make_cache(cfg, n=n0, extra=steps + 4, splits=splits) for _ in range(2)]
    eager, graphed = caches
    try:
        print(f"graph test: {cfg.name} batch={cfg.batch} n0={n0} layers={layers} splits={graphed.splits}",
              flush=True)
        assert graphed.splits == splits
        lays = {l: gen_layer(cfg, l, n=n0) for l in layers}
        for c in caches:
            G.load_bases(c, bases, groups=groups)
            for l in layers:
                G.load_layer(c, l, lays[l])
        B, Hq, Hkv, d = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
        dev = torch.device("cuda")
        sq = [torch.zeros((B, Hq, d), dtype=torch.float16, device=dev) for _ in layers]
        sk = [torch.zeros((B, Hkv, d), dtype=torch.float16, device=dev) for _ in layers]
        sv = [torch.zeros((B, Hkv, d), dtype=torch.float16, device=dev) for _ in layers]
        st = [torch.zeros((B, Hkv), dtype=torch.uint8, device=dev) for _ in layers]
        so = [torch.zeros((B, Hq, d), dtype=torch.float32, device=dev) for _ in layers]
        graphed.workspace(B)          # allocated before capture, its counters zero
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i, l in enumerate(layers):
                graphed.decode_step(l, sq[i], sk[i], sv[i], st[i], out=so[i])
        torch.cuda.synchronize()

        for step in range(steps):
            # eager work of the program's own on the graph's cache, through the
            # workspace the graph's launches use: a decode of the first layer,
            # both caches as the previous step left them
            q0 = G.dev(gen_query(cfg, layers[0], step=100 + step))
            mid_e = eager.decode(layers[0], q0)
            mid_g = graphed.decode(layers[0], q0)
            outs = []
            for i, l in enumerate(layers):
                q = gen_query(cfg, l, step=step)
                a = gen_append_inputs(cfg, l, step, bases)
                outs.append(eager.decode_step(l, G.dev(q), G.dev(a["k"]), G.dev(a["v"]), G.dev(a["tier"])))
                sq[i].copy_(G.dev(q))
                sk[i].copy_(G.dev(a["k"]))
                sv[i].copy_(G.dev(a["v"]))
                st[i].copy_(G.dev(a["tier"]))
                if step == 0 and i == 0:
                    torch.cuda.synchronize()
                    m = l // cfg.layers_per_group
                    ref = oracle.decode(cfg, lays[l], bases["K"][m], bases["V"][m], q)
                    err = G.norm_err(outs[0].cpu().numpy().astype(np.float64), ref)
                    assert err.max() <= TOL, f"eager step against the oracle: {err.max():.3e}"
            g.replay()
            torch.cuda.synchronize()
            for i, l in enumerate(layers):
                assert np.array_equal(_bits(so[i]), _bits(outs[i])), f"step {step} layer {l}: replay differs"
            assert np.array_equal(_bits(mid_g), _bits(mid_e)), f"step {step}: eager decode between replays differs"
            print(f"  step {step}: {len(layers)} replayed launches equal the eager ones", flush=True)

        for l in layers:
            n_max = n0 + steps
            ex_e, cnt_e, sl_e = G.export_np(eager, l, B, n_max)
            ex_g, cnt_g, sl_g = G.export_np(graphed, l, B, n_max)
            assert np.array_equal(cnt_e, cnt_g) and np.array_equal(sl_e, sl_g), f"layer {l}: counts or slots"
            assert int(cnt_g.sum()) == B * Hkv * (n0 + steps)
            for key in ex_e:
                assert np.array_equal(ex_e[key].view(np.uint8), ex_g[key].view(np.uint8)), (l, key)
        for c in caches:
            assert c.check_errors() == 0
        del g
    finally:
        for c in caches:
            c.close()


def test_decode_attn_graph_replays_follow_the_query_buffer(G):
    """A captured dwkv_decode_attn (it leaves the cache unchanged): three
    replays with different queries written into its buffer, each equal bit
    for bit to an eager decode of the same query, with eager decodes of other
    queries between the replays."""
    import torch
    cfg = w.get_config(1)
    layer, n0 = 3, 8192
    bases = make_bases(cfg)
    m = layer // cfg.layers_per_group
    cache = G.make_cache(cfg, n=n0, splits=32)
    try:
        print(f"graph test: decode_attn {cfg.name} n0={n0} splits={cache.splits}", flush=True)
        G.load_bases(cache, bases, groups=[m])
        G.load_layer(cache, layer, gen_layer(cfg, layer, n=n0))
        B, Hq, d = cfg.batch, cfg.num_q_heads, cfg.head_dim
        sq = torch.zeros((B, Hq, d), dtype=torch.float16, device="cuda")
        so = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
        cache.workspace(B)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cache.decode(layer, sq, out=so)
        torch.cuda.synchronize()
        for rep in range(3):
            q = G.dev(gen_query(cfg, layer, step=rep))
            want = cache.decode(layer, q)
            other = cache.decode(layer, G.dev(gen_query(cfg, layer, step=50 + rep)))
            sq.copy_(q)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(_bits(so), _bits(want)), f"replay {rep} differs from the eager decode"
            assert not np.array_equal(_bits(other), _bits(want))
            print(f"  replay {rep}: equal to the eager decode", flush=True)
        assert cache.check_errors() == 0
        del g
    finally:
        cache.close()
