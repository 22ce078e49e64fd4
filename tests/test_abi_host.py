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


def test_tier_table_validation():
    assert _rc_arena(_cfg(tier_rank=(8, 8, 32, 64))) == d.DWKV_ERR_INVALID_ARG      # not ascending
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
    bases = 8 * 3 * 8 * 64 * 128 * 2       # K and V bases, and a transposed copy of V
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
