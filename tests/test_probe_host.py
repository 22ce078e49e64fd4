"""dwkv_probe_update (the host-side threshold feedback after the paper's
Eq. (3)) against oracle.probe_controller, bit for bit in fp32, and the
probe's host argument checks (CPU, no GPU)."""
import ctypes

import numpy as np
import pytest

import compressed_kv_cache_dwkv_amd as d
import oracle


@pytest.mark.parametrize("seed", range(5))
def test_controller_matches_oracle_bit_for_bit(seed):
    rng = np.random.default_rng(seed)
    W = 8
    tol, step, patience, lo, hi = 0.03, 0.0625 if seed % 2 else 0.05, 1 + seed % 4, 0.1, 0.9
    tau = rng.uniform(lo, hi, W).astype(np.float32)
    below = np.zeros(W, np.int32)
    ref_tau = [float(t) for t in tau]
    ref_below = [0] * W
    for it in range(60):
        err = (rng.exponential(0.03, W)).astype(np.float32)
        d.dwkv_probe_update(tau, below, err, tol, step, patience, lo, hi)
        for m in range(W):
            ref_tau[m], ref_below[m] = oracle.probe_controller(ref_tau[m], ref_below[m], float(err[m]), tol, step,
                                                               patience, lo, hi)
        assert np.array_equal(tau, np.asarray(ref_tau, np.float32)), it
        assert list(below) == ref_below


def test_controller_and_probe_reject_bad_arguments():
    L = d._lib
    tau = np.zeros(2, np.float32)
    below = np.zeros(2, np.int32)
    err = np.zeros(2, np.float32)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert L.dwkv_probe_update(P(tau), P(below), 0, P(err), 0.1, 0.1, 1, 0.0, 1.0) == d.DWKV_ERR_INVALID_ARG
    assert L.dwkv_probe_update(P(tau), P(below), 2, P(err), 0.1, 0.1, 0, 0.0, 1.0) == d.DWKV_ERR_INVALID_ARG
    assert L.dwkv_probe_update(P(tau), P(below), 2, P(err), 0.1, 0.1, 1, 1.0, 0.0) == d.DWKV_ERR_INVALID_ARG
    assert L.dwkv_probe_update(None, P(below), 2, P(err), 0.1, 0.1, 1, 0.0, 1.0) == d.DWKV_ERR_INVALID_ARG
    cfg = d.make_config(4, 2, 8, 2, 64, 32, (8, 16, 32), (4, 4, 4), 4, 2, (100, 50, 20), 170, 0)
    h = ctypes.c_void_p()
    assert L.dwkv_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 40), d.dwkv_arena_bytes(cfg), ctypes.byref(h)) == d.DWKV_OK
    try:
        kk = ctypes.c_void_p(1 << 44)
        ws = d.dwkv_probe_workspace_bytes(cfg, 2, 3, 4)
        wsp = ctypes.c_void_p(1 << 43)
        call = lambda **kw: L.dwkv_probe_error(h, kw.get("layer", 0), kk, kw.get("nq", 3), kw.get("B", 2), kk, kk, kk,
                                               kw.get("n_cap", 192), kw.get("S", 4), kw.get("sc", 0.1), 1e-6, kk,
                                               wsp, kw.get("ws", ws), None)
        assert call(layer=4) == d.DWKV_ERR_INVALID_ARG
        assert call(nq=0) == d.DWKV_ERR_INVALID_ARG
        assert call(B=3) == d.DWKV_ERR_INVALID_ARG
        assert call(n_cap=100) == d.DWKV_ERR_INVALID_ARG
        assert call(S=0) == d.DWKV_ERR_INVALID_ARG
        assert call(sc=-1.0) == d.DWKV_ERR_INVALID_ARG
        assert call(ws=ws - 1) == d.DWKV_ERR_WORKSPACE
    finally:
        L.dwkv_destroy(h)
