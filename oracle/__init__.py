"""CPU oracle for the DepthWeave-KV decode path -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The product (compressed_kv_cache_dwkv_amd) never does.  It
shares no code with the HIP library; see oracle.c for what each entry point
computes and the passage it follows.

Pins (tests/test_oracle_*.py): fp16 codec exhaustively against NumPy; decode
against torch's scaled_dot_product_attention in fp64 on identity bases,
closed forms (one token, two tokens, zero query, constant values, zero token),
permutation / linearity / grouping invariants and planted needles; append
against hand-computable identity and signed-permutation bases, brute-force
best s-subset, quantisation bounds and tie rules.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class _Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("r_max", ctypes.c_int32), ("s_max", ctypes.c_int32),
        ("n_max", ctypes.c_int64), ("num_tiers", ctypes.c_int32),
        ("tier_rank", ctypes.c_int32 * 8), ("tier_resid", ctypes.c_int32 * 8),
    ]


def _load(path: str):
    """Open a build of oracle.c and declare its entry points."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.oracle_half_to_double.restype = ctypes.c_double
    L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    L.oracle_float_to_half.restype = ctypes.c_uint16
    L.oracle_float_to_half.argtypes = [ctypes.c_float]
    L.oracle_half_to_double_array.argtypes = [P, P, ctypes.c_int64]
    L.oracle_float_to_half_array.argtypes = [P, P, ctypes.c_int64]
    L.oracle_decode.restype = ctypes.c_int
    L.oracle_decode.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, P, P, P, P, P, P, P,
                                P, ctypes.c_double, P, P, ctypes.c_int, ctypes.c_int]
    L.oracle_append.restype = ctypes.c_int
    L.oracle_append.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_uint16, P, P, P, P]
    L.oracle_append_residual.restype = ctypes.c_int
    L.oracle_append_residual.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, P]
    L.oracle_max_threads.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build
            build()
        _lib = _load(_LIB_PATH)
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    assert a.dtype == np.uint16
    return a


# ------------------------------------------------------------------ fp16 codec
def half_to_double(h) -> np.ndarray:
    h = _u16(np.asarray(h))
    out = np.empty(h.shape, np.float64)
    lib().oracle_half_to_double_array(_p(h), _p(out), h.size)
    return out


def float_to_half(f) -> np.ndarray:
    """fp32 -> fp16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().oracle_float_to_half_array(_p(f), _p(out), f.size)
    return out


# ------------------------------------------------------------------ decode
def max_threads() -> int:
    return int(lib().oracle_max_threads())


def decode(cfg, lay: Dict[str, np.ndarray], basisK: np.ndarray, basisV: np.ndarray,
           q: np.ndarray, alpha: Optional[float] = None,
           pairs: Optional[Sequence[Sequence[int]]] = None, threads: int = 0,
           tier_resid: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention output [B][H_q][d] (fp64) of one layer.

    lay: logical layer (workload.gen_layer format); basisK/V: fp16
    [H_kv][r_max][d] of the layer's depth group; q: fp16 [B][H_q][d].
    alpha defaults to 1/sqrt(d).  pairs: optional list of (b, kv_head) to
    compute (other rows are returned as NaN)."""
    B, Hkv, n_max, R = lay["coefK"].shape
    Hq, d = q.shape[1], q.shape[2]
    S = lay["idxK"].shape[3]
    sh = _Shape()
    sh.batch, sh.num_q_heads, sh.num_kv_heads, sh.head_dim = B, Hq, Hkv, d
    sh.r_max, sh.s_max, sh.n_max = R, S, n_max
    sh.num_tiers = cfg.num_tiers
    res = tuple(tier_resid) if tier_resid is not None else cfg.resid_per_tier
    for k in range(cfg.num_tiers):
        sh.tier_rank[k] = cfg.tier_rank[k]
        sh.tier_resid[k] = res[k]
    if alpha is None:
        alpha = 1.0 / np.sqrt(d)
    out = np.full((B, Hq, d), np.nan, np.float64)
    if pairs is None:
        pa, npairs = None, 0
    else:
        parr = np.ascontiguousarray(np.asarray(pairs, np.int32).reshape(-1, 2))
        pa, npairs = _p(parr), parr.shape[0]
    c = {k: np.ascontiguousarray(v) for k, v in lay.items()}
    rc = lib().oracle_decode(
        ctypes.byref(sh), _p(np.ascontiguousarray(c["n_tokens"], np.int64)), _p(c["tier"]),
        _p(_u16(basisK)), _p(_u16(basisV)), _p(_u16(c["coefK"])), _p(_u16(c["coefV"])),
        _p(c["idxK"]), _p(c["idxV"]), _p(c["valK"]), _p(c["valV"]),
        _p(_u16(c["scaleK"])), _p(_u16(c["scaleV"])), _p(_u16(q)), float(alpha), _p(out),
        pa, npairs, int(threads))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return out


# ------------------------------------------------------------------ append
def append_vector(basis: np.ndarray, x: np.ndarray, r: int, s: int, qmax: int,
                  gate: Optional[np.float16] = None):
    """Encode one fp16 vector.  basis: fp16 [r_max][d]; x: fp16 [d].
    Returns (c fp16[r], idx uint8[s], val int8[s], scale fp16)."""
    b = _u16(basis)
    xv = _u16(x)
    r_max, d = b.shape
    c = np.zeros(max(r, 1), np.uint16)
    idx = np.zeros(max(s, 1), np.uint8)
    val = np.zeros(max(s, 1), np.int8)
    sc = np.zeros(1, np.uint16)
    g = 0x3C00 if gate is None else int(np.asarray(gate, np.float16).view(np.uint16))
    rc = lib().oracle_append(d, r_max, _p(b), _p(xv), r, s, qmax, g, _p(c), _p(idx), _p(val), _p(sc))
    if rc != 0:
        raise ValueError("oracle_append rejected its arguments")
    return c[:r].view(np.float16), idx[:s], val[:s], sc.view(np.float16)[0]


def append_residual(basis: np.ndarray, x: np.ndarray, r: int) -> np.ndarray:
    """fp32 residual e = x - B^T fp16(B x) of the encoder (step 2)."""
    b = _u16(basis)
    xv = _u16(x)
    r_max, d = b.shape
    e = np.zeros(d, np.float32)
    if lib().oracle_append_residual(d, r_max, _p(b), _p(xv), r, _p(e)) != 0:
        raise ValueError("oracle_append_residual rejected its arguments")
    return e


def append_layer(cfg, basisK: np.ndarray, basisV: np.ndarray, k: np.ndarray, v: np.ndarray,
                 tier: np.ndarray, gateK: Optional[np.ndarray] = None,
                 gateV: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Encode the new token of every (b, KV head) of one layer.

    k, v: fp16 [B][H_kv][d]; tier: uint8 [B][H_kv]; gateK, gateV: optional
    fp16 [B][H_kv] (None = a gate of 1).  Returns logical-token arrays: coef{K,V} [B][H_kv][r_max] fp16
    (zero beyond the rank), idx/val{K,V} [B][H_kv][s_max], scale{K,V} [B][H_kv]."""
    B, H, d = k.shape
    R, S = cfg.r_max, cfg.s_max
    res = cfg.resid_per_tier
    out = {}
    for z, x, bas, gate in (("K", k, basisK, gateK), ("V", v, basisV, gateV)):
        coef = np.zeros((B, H, R), np.float16)
        idx = np.zeros((B, H, S), np.uint8)
        val = np.zeros((B, H, S), np.int8)
        sc = np.zeros((B, H), np.float16)
        for b in range(B):
            for h in range(H):
                t = int(tier[b, h])
                r, s = cfg.tier_rank[t], res[t]
                g = None if gate is None else gate[b, h]
                c, i, vv, scale = append_vector(bas[h], x[b, h], r, s, cfg.qmax, g)
                coef[b, h, :r] = c
                idx[b, h, :s] = i
                val[b, h, :s] = vv
                sc[b, h] = scale
        out["coef" + z], out["idx" + z], out["val" + z], out["scale" + z] = coef, idx, val, sc
    return out
