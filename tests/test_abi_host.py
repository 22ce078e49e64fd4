"""C ABI host logic (CPU, no GPU call): the library loads, exports every
declared entry point, and rejects bad arguments before queuing any work."""
import ctypes

import pytest

import compressed_kv_cache_dwkv_amd as d
import workload as w


def _cfg(**kw):
    base = dict(num_layers=32, layers_per_group=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                r_max=64, tier_rank=(8, 16, 32, 64), tier_resid=(8, 8, 8, 8), resid_bits=4,
                max_batch=2, tier_capacity=(100, 50, 25, 16), max_tokens=191, decode_splits=0)
    base.update(kw)
    return d.make_config(**base)


def _rc_arena(cfg):
    n = ctypes.c_size_t()
    return d._lib.dwkv_arena_bytes(ctypes.byref(cfg), ctypes.byref(n))


def test_every_declared_symbol_is_exported():
    syms = d.declared_symbols()
    assert len(syms) >= 14
    for s in syms:
        assert hasattr(d._lib, s), s
        assert callable(getattr(d._lib, s))


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, d.DWKV_ERR_UNSUPPORTED),
    ("r_max", 130, d.DWKV_ERR_UNSUPPORTED),
    ("r_max", 62, d.DWKV_ERR_UNSUPPORTED),
    ("resid_bits", 2, d.DWKV_ERR_UNSUPPORTED),
    ("num_q_heads", 24, d.DWKV_ERR_UNSUPPORTED),      # 3 query heads per KV head
    ("num_q_heads", 30, d.DWKV_ERR_INVALID_ARG),      # not a multiple
    ("num_layers", 0, d.DWKV_ERR_INVALID_ARG),
    ("max_batch", 0, d.DWKV_ERR_INVALID_ARG),
    ("decode_splits", -1, d.DWKV_ERR_INVALID_ARG),
    ("decode_splits", 257, d.DWKV_ERR_UNSUPPORTED),
])
def test_config_validation(field, value, code):
    cfg = _cfg()
    setattr(cfg, field, value)
    assert _rc_arena(cfg) == code


def test_coefficient_form_validation_and_size():
    """coef_bits 16 (or 0) and 8; 8-bit codes only with bases of at most 64
    vectors; the 8-bit arena holds r + 2 bytes per token and Z instead of 2 r."""
    assert _rc_arena(_cfg(coef_bits=7)) == d.DWKV_ERR_UNSUPPORTED
    assert _rc_arena(_cfg(coef_bits=8, r_max=128, tier_rank=(8, 16, 32, 128))) == d.DWKV_ERR_UNSUPPORTED
    cap = (40000, 20000, 10000, 7000)
    a16 = d.dwkv_arena_bytes(_cfg(tier_capacity=cap, max_tokens=1, max_batch=1))
    a8 = d.dwkv_arena_bytes(_cfg(tier_capacity=cap, max_tokens=1, max_batch=1, coef_bits=8))
    saved = 32 * 8 * sum(c * (2 * 2 * r - (2 * r + 4)) for c, r in zip(cap, (8, 16, 32, 64)))
    assert abs((a16 - a8) - saved) <= 32 * 8 * 2048        # per-array alignment of the head blocks


def test_tier_table_validation():
    assert _rc_arena(_cfg(tier_rank=(16, 8, 32, 64))) == d.DWKV_ERR_INVALID_ARG     # descending
    assert _rc_arena(_cfg(tier_rank=(16, 16, 16, 16), tier_resid=(0, 2, 4, 8))) == d.DWKV_OK   # fixed r_b, routed s
    assert _rc_arena(_cfg(tier_rank=(8, 16, 32, 72))) == d.DWKV_ERR_UNSUPPORTED     # above r_max
    assert _rc_arena(_cfg(tier_rank=(6, 16, 32, 64))) == d.DWKV_ERR_UNSUPPORTED     # not /4
    assert _rc_arena(_cfg(tier_resid=(8, 8, 8, 9))) == d.DWKV_ERR_UNSUPPORTED
    cfg = _cfg()
    cfg.num_tiers = 9
    assert _rc_arena(cfg) == d.DWKV_ERR_UNSUPPORTED
    assert _rc_arena(_cfg(tier_resid=(0, 2, 4, 8))) == d.DWKV_OK


def test_arena_holds_every_algorithmic_byte_with_small_overhead():
    c = w.get_config(2)
    cap = [40000, 20000, 10000, 7000]
    cfg = _cfg(tier_capacity=cap, max_tokens=70000, max_batch=1)
    total = d.dwkv_arena_bytes(cfg)
    per_head = sum(k * w.compressed_bytes_per_token(r, 8, 4) for k, r in zip(cap, c.tier_rank))
    heads = 32 * 8
    bases = 8 * 4 * 8 * 64 * 128 * 2       # K and V bases, and transposed copies of both
    posmap = heads * 70000 * 4
    assert total >= heads * per_head + bases + posmap
    assert total <= heads * per_head * 1.001 + bases + posmap + heads * 4 * 4 + 65536


def test_create_and_call_validation_without_gpu():
    cfg = _cfg()
    need = d.dwkv_arena_bytes(cfg)
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(1 << 40)   # never dereferenced by host-only paths
    assert d._lib.dwkv_create(ctypes.byref(cfg), None, need, ctypes.byref(h)) == d.DWKV_ERR_INVALID_ARG
    assert d._lib.dwkv_create(ctypes.byref(cfg), ctypes.c_void_p((1 << 40) + 16), need,
                              ctypes.byref(h)) == d.DWKV_ERR_INVALID_ARG
    assert d._lib.dwkv_create(ctypes.byref(cfg), fake, need - 1, ctypes.byref(h)) == d.DWKV_ERR_WORKSPACE
    assert d._lib.dwkv_create(ctypes.byref(cfg), fake, need, ctypes.byref(h)) == d.DWKV_OK
    try:
        ws = d.dwkv_workspace_bytes(cfg, 2)
        q = ctypes.c_void_p(1 << 41)
        out = ctypes.c_void_p(1 << 42)
        wsp = ctypes.c_void_p(1 << 43)
        L = d._lib
        # decode: layer, batch, scale, workspace size/alignment, nulls
        assert L.dwkv_decode_attn(h, 32, q, 1, 0.1, out, wsp, ws, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_attn(h, -1, q, 1, 0.1, out, wsp, ws, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_attn(h, 0, q, 3, 0.1, out, wsp, ws, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_attn(h, 0, q, 1, 0.0, out, wsp, ws, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_attn(h, 0, q, 1, float("nan"), out, wsp, ws, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_attn(h, 0, q, 2, 0.1, out, wsp, ws - 1, None) == d.DWKV_ERR_WORKSPACE
        assert L.dwkv_decode_attn(h, 0, None, 1, 0.1, out, wsp, ws, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_attn(h, 0, q, 1, 0.1, out, ctypes.c_void_p((1 << 43) + 8), ws,
                                  None) == d.DWKV_ERR_INVALID_ARG
        # fused step: the decode checks plus the append inputs
        kk = ctypes.c_void_p(1 << 44)
        assert L.dwkv_decode_step(h, 0, q, 1, 0.1, out, wsp, ws, None, kk, kk, None, None,
                                  None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_step(h, 0, q, 1, 0.1, out, wsp, ws, kk, kk, None, None, None,
                                  None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_step(h, 32, q, 1, 0.1, out, wsp, ws, kk, kk, kk, None, None,
                                  None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_step(h, 0, q, 1, 0.0, out, wsp, ws, kk, kk, kk, None, None,
                                  None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_step(h, 0, q, 2, 0.1, out, wsp, ws - 1, kk, kk, kk, None, None,
                                  None) == d.DWKV_ERR_WORKSPACE
        assert L.dwkv_decode_step(h, 0, q, 1, 0.1, out, ctypes.c_void_p((1 << 43) + 8), ws, kk, kk, kk,
                                  None, None, None) == d.DWKV_ERR_INVALID_ARG
        # append
        assert L.dwkv_append(h, 0, q, None, q, None, None, 1, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_append(h, 40, q, q, q, None, None, 1, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_append(h, 0, q, q, q, None, None, 0, None) == d.DWKV_ERR_INVALID_ARG
        # import: capacity and n_max checks happen on the host
        lay = d.dwkv_logical_layer()
        lay.n_max = 500
        for f in ("tier", "coefK", "coefV", "idxK", "idxV", "valK", "valV", "scaleK", "scaleV"):
            setattr(lay, f, 1 << 44)
        n = (ctypes.c_int64 * 2)(192, 10)
        assert L.dwkv_import_layer(h, 0, ctypes.byref(lay), n, 2, None) == d.DWKV_ERR_CAPACITY
        n = (ctypes.c_int64 * 2)(501, 10)
        assert L.dwkv_import_layer(h, 0, ctypes.byref(lay), n, 2, None) == d.DWKV_ERR_INVALID_ARG
        lay.valV = None
        n = (ctypes.c_int64 * 2)(5, 10)
        assert L.dwkv_import_layer(h, 0, ctypes.byref(lay), n, 2, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_set_basis(h, 8, q, q, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_read_counts(h, 0, 3, q, None) == d.DWKV_ERR_INVALID_ARG
    finally:
        assert d._lib.dwkv_destroy(h) == d.DWKV_OK
    assert d._lib.dwkv_destroy(None) == d.DWKV_ERR_INVALID_ARG


@pytest.mark.parametrize("ci,extra,expect", [(1, 282, 9), (2, 282, 32), (3, 82, 2), (4, 82, 32), (2, 6, 32),
                                             (4, 6, 32)])
def test_split_plan_of_the_workloads(ci, extra, expect):
    """The split count the benchmark's caches get (capacities of the
    workload plus its appended tokens) and the full-size step tests' (a few
    spare slots) agree: 32 at 64K and 128K."""
    from workload.gen import max_tier_counts
    c = w.get_config(ci)
    cap = [int(x) + extra for x in max_tier_counts(c)]
    cfg = d.make_config(c.num_layers, c.layers_per_group, c.num_q_heads, c.num_kv_heads, c.head_dim,
                        c.r_max, c.tier_rank, c.resid_per_tier, c.resid_bits, c.batch, cap,
                        c.n_tokens + extra, 0)
    h = ctypes.c_void_p()
    need = d.dwkv_arena_bytes(cfg)
    assert d._lib.dwkv_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 40), need, ctypes.byref(h)) == d.DWKV_OK
    try:
        assert d.dwkv_decode_splits(h) == expect
    finally:
        d._lib.dwkv_destroy(h)
    n = ctypes.c_int()
    assert d._lib.dwkv_decode_splits(None, ctypes.byref(n)) == d.DWKV_ERR_INVALID_ARG


def test_noalloc_step_rejects_what_its_scratch_cannot_hold():
    """Host checks of dwkv_decode_step_noalloc, before any HIP call: more
    (sequence, KV head) pairs than its counters, or partials larger than its
    static array, give DWKV_ERR_WORKSPACE; bad arguments INVALID_ARG."""
    L = d._lib
    kk = ctypes.c_void_p(1 << 44)
    big = _cfg(max_batch=200, decode_splits=8)           # 200 x 8 pairs > 1024
    h = ctypes.c_void_p()
    assert L.dwkv_create(ctypes.byref(big), ctypes.c_void_p(1 << 40), d.dwkv_arena_bytes(big),
                         ctypes.byref(h)) == d.DWKV_OK
    try:
        assert L.dwkv_decode_step_noalloc(h, 0, kk, 129, 0.1, kk, kk, kk, kk, None, None,
                                          None) == d.DWKV_ERR_WORKSPACE
        assert L.dwkv_decode_step_noalloc(h, 0, kk, 201, 0.1, kk, kk, kk, kk, None, None,
                                          None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_step_noalloc(h, 0, kk, 1, 0.1, kk, kk, None, kk, None, None,
                                          None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_step_noalloc(h, 32, kk, 1, 0.1, kk, kk, kk, kk, None, None,
                                          None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_decode_step_noalloc(h, 0, kk, 1, 0.0, kk, kk, kk, kk, None, None,
                                          None) == d.DWKV_ERR_INVALID_ARG
    finally:
        L.dwkv_destroy(h)
    wide = _cfg(max_batch=16, decode_splits=256)          # 16 x 32 x 256 x 128 x 4 B of partials
    assert L.dwkv_create(ctypes.byref(wide), ctypes.c_void_p(1 << 40), d.dwkv_arena_bytes(wide),
                         ctypes.byref(h)) == d.DWKV_OK
    try:
        assert L.dwkv_decode_step_noalloc(h, 0, kk, 16, 0.1, kk, kk, kk, kk, None, None,
                                          None) == d.DWKV_ERR_WORKSPACE
    finally:
        L.dwkv_destroy(h)


def test_dense_comparator_host_checks():
    """dwkv_dense_decode / dwkv_materialize_layer reject bad shapes before
    any HIP call."""
    L = d._lib
    kk = ctypes.c_void_p(1 << 44)
    ws = d.dwkv_dense_workspace_bytes(2, 32, 8, 128, 16)
    assert ws >= 2 * 32 * 16 * 128 * 4
    n = ctypes.c_size_t()
    assert L.dwkv_dense_workspace_bytes(2, 24, 8, 128, 16, ctypes.byref(n)) == d.DWKV_ERR_INVALID_ARG
    assert L.dwkv_dense_workspace_bytes(2, 32, 8, 96, 16, ctypes.byref(n)) == d.DWKV_ERR_INVALID_ARG
    assert L.dwkv_dense_workspace_bytes(2, 32, 8, 128, 0, ctypes.byref(n)) == d.DWKV_ERR_INVALID_ARG
    wsp = ctypes.c_void_p(1 << 43)
    args = dict(q=kk, k=kk, v=kk, n=kk, B=2, Hq=32, Hkv=8, d=128, n_cap=4096, S=16, sc=0.1, out=kk)
    def call(**kw):
        a = dict(args, **kw)
        return L.dwkv_dense_decode(a["q"], a["k"], a["v"], a["n"], a["B"], a["Hq"], a["Hkv"], a["d"], a["n_cap"],
                                   a["S"], a["sc"], a["out"], kw.get("wsp", wsp), kw.get("ws", ws), None)
    assert call(q=None) == d.DWKV_ERR_INVALID_ARG
    assert call(n_cap=4000) == d.DWKV_ERR_INVALID_ARG          # not a multiple of 64
    assert call(sc=0.0) == d.DWKV_ERR_INVALID_ARG
    assert call(S=257) == d.DWKV_ERR_INVALID_ARG
    assert call(ws=ws - 1) == d.DWKV_ERR_WORKSPACE
    assert call(wsp=ctypes.c_void_p((1 << 43) + 8)) == d.DWKV_ERR_INVALID_ARG
    cfg = _cfg()
    h = ctypes.c_void_p()
    assert L.dwkv_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 40), d.dwkv_arena_bytes(cfg), ctypes.byref(h)) == d.DWKV_OK
    try:
        assert L.dwkv_materialize_layer(h, 0, 1, kk, None, 256, None, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_materialize_layer(h, 32, 1, kk, kk, 256, None, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_materialize_layer(h, 0, 3, kk, kk, 256, None, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_materialize_layer(h, 0, 1, kk, kk, 128, None, None) == d.DWKV_ERR_INVALID_ARG   # < max_tokens
        assert L.dwkv_materialize_layer(h, 0, 1, kk, kk, 200, None, None) == d.DWKV_ERR_INVALID_ARG   # not /64
    finally:
        L.dwkv_destroy(h)


def test_prefill_host_checks():
    """The prefill entry points reject bad arguments before any HIP call; the
    workspace starts with the fp64 Gram sums of every window."""
    L = d._lib
    cfg = _cfg()
    ws = d.dwkv_prefill_workspace_bytes(cfg)
    assert ws >= 8 * 2 * 8 * 128 * 128 * 8
    h = ctypes.c_void_p()
    assert L.dwkv_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 40), d.dwkv_arena_bytes(cfg), ctypes.byref(h)) == d.DWKV_OK
    kk = ctypes.c_void_p(1 << 44)
    wsp = ctypes.c_void_p(1 << 43)
    try:
        g = lambda layer=0, k=kk, v=kk, n=kk, B=1, cap=4096, p=wsp, sz=ws: L.dwkv_prefill_gram(
            h, layer, k, v, n, B, cap, 1, p, sz, None)
        assert g(k=None) == d.DWKV_ERR_INVALID_ARG
        assert g(n=None) == d.DWKV_ERR_INVALID_ARG
        assert g(layer=32) == d.DWKV_ERR_INVALID_ARG
        assert g(B=0) == d.DWKV_ERR_INVALID_ARG
        assert g(B=3) == d.DWKV_ERR_INVALID_ARG                     # more than max_batch
        assert g(cap=0) == d.DWKV_ERR_INVALID_ARG
        assert g(k=ctypes.c_void_p((1 << 44) + 8)) == d.DWKV_ERR_INVALID_ARG
        assert g(p=ctypes.c_void_p((1 << 43) + 64)) == d.DWKV_ERR_INVALID_ARG
        assert g(sz=ws - 1) == d.DWKV_ERR_WORKSPACE
        assert g(cap=(1 << 24)) == d.DWKV_ERR_UNSUPPORTED              # rows beyond 32-bit byte offsets
        b = lambda g0=0, ng=1, om=kk, k=72, q=2, sz=ws: L.dwkv_prefill_bases(h, g0, ng, om, k, q, None, wsp, sz, None)
        assert b(om=None) == d.DWKV_ERR_INVALID_ARG
        assert b(g0=7, ng=2) == d.DWKV_ERR_INVALID_ARG
        assert b(ng=0) == d.DWKV_ERR_INVALID_ARG
        assert b(k=60) == d.DWKV_ERR_INVALID_ARG                   # narrower than r_max
        assert b(k=129) == d.DWKV_ERR_INVALID_ARG                  # wider than head_dim
        assert b(k=80) == d.DWKV_ERR_UNSUPPORTED                   # beyond the LDS-resident sketch
        assert b(q=-1) == d.DWKV_ERR_INVALID_ARG
        assert b(sz=ws - 1) == d.DWKV_ERR_WORKSPACE
        assert L.dwkv_prefill_encode(h, 0, kk, kk, kk, 1, 4096, None, None, None, wsp, ws, None) == d.DWKV_ERR_INVALID_ARG
        assert L.dwkv_prefill_encode(h, 0, kk, kk, kk, 1, 4096, kk, None, None, wsp, ws - 1,
                                     None) == d.DWKV_ERR_WORKSPACE
    finally:
        L.dwkv_destroy(h)


def test_workspace_scales_with_batch_and_splits():
    a = d.dwkv_workspace_bytes(_cfg(decode_splits=4), 1)
    b = d.dwkv_workspace_bytes(_cfg(decode_splits=8), 1)
    c = d.dwkv_workspace_bytes(_cfg(decode_splits=8), 2)
    assert a < b < c
    assert d.dwkv_workspace_bytes(_cfg(decode_splits=8), 1) >= 32 * 8 * 128 * 4


def test_strerror():
    assert d.dwkv_strerror(0) == "ok"
    for code in range(-6, 0):
        assert d.dwkv_strerror(code) != "unknown error"
    assert d.dwkv_strerror(-99) == "unknown error"


def test_single_hip_runtime_in_process():
    """The binding must share torch's HIP runtime: one libamdhip64 mapped."""
    maps = open("/proc/self/maps").read()
    libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(libs) == 1, libs


def test_stream_probe_validation_without_gpu():
    """The streaming-read probe refuses bad pointers, sizes and grids before
    any device call (fake, aligned device addresses: nothing is launched)."""
    L = d._lib
    src, sink = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    ok = dict(bytes=1 << 16, wg=256, th=512)
    assert L.dwkv_stream_probe(None, ok["bytes"], ok["wg"], ok["th"], 0, sink, None) == d.DWKV_ERR_INVALID_ARG
    assert L.dwkv_stream_probe(src, ok["bytes"], ok["wg"], ok["th"], 0, None, None) == d.DWKV_ERR_INVALID_ARG
    assert L.dwkv_stream_probe(ctypes.c_void_p((1 << 20) + 8), ok["bytes"], ok["wg"], ok["th"], 0, sink,
                               None) == d.DWKV_ERR_INVALID_ARG
    for nbytes in (0, -16, 24):
        assert L.dwkv_stream_probe(src, nbytes, ok["wg"], ok["th"], 0, sink, None) == d.DWKV_ERR_INVALID_ARG
    for wg, th in ((0, 512), (65536, 512), (256, 0), (256, 96), (256, 2048)):
        assert L.dwkv_stream_probe(src, ok["bytes"], wg, th, 0, sink, None) == d.DWKV_ERR_INVALID_ARG


@pytest.mark.parametrize("n,expect", [(8192, 8), (16384, 16), (32768, 32), (131072, 32)])
def test_split_plan_over_context(n, expect):
    """The Llama-3-8B shape at batch 1 and other contexts, with the spare
    slots of `bench.py --context n --steps 64` (8 warm-up steps, 64 timed,
    10 kernel repetitions, 8 more): one split per 1024 token slots until
    every compute unit has a workgroup (32 splits of 8 KV heads), as the
    context sweep ran them."""
    from workload.gen import max_tier_counts
    c = w.get_config(2).with_(n_tokens=n)
    extra = 8 + 64 + 10 + 8
    cap = [int(x) + extra for x in max_tier_counts(c)]
    cfg = d.make_config(c.num_layers, c.layers_per_group, c.num_q_heads, c.num_kv_heads, c.head_dim,
                        c.r_max, c.tier_rank, c.resid_per_tier, c.resid_bits, c.batch, cap,
                        c.n_tokens + extra, 0)
    h = ctypes.c_void_p()
    need = d.dwkv_arena_bytes(cfg)
    assert d._lib.dwkv_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 40), need, ctypes.byref(h)) == d.DWKV_OK
    try:
        assert d.dwkv_decode_splits(h) == expect
    finally:
        d._lib.dwkv_destroy(h)
