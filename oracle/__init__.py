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
        ("coef_bits", ctypes.c_int32),
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
    L.oracle_decode.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                P, ctypes.c_double, P, P, ctypes.c_int, ctypes.c_int]
    L.oracle_materialize.restype = ctypes.c_int
    L.oracle_materialize.argtypes = [ctypes.POINTER(_Shape), P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                     ctypes.c_int]
    L.oracle_dense_decode.restype = ctypes.c_int
    L.oracle_dense_decode.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                      P, P, P, P, ctypes.c_double, P, ctypes.c_int]
    L.oracle_append_ex.restype = ctypes.c_int
    L.oracle_append_ex.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_uint16, ctypes.c_int, P, P, P, P, P]
    L.oracle_append.restype = ctypes.c_int
    L.oracle_append.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int,
                                ctypes.c_int, ctypes.c_uint16, P, P, P, P]
    L.oracle_append_residual.restype = ctypes.c_int
    L.oracle_append_residual.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, P]
    L.oracle_append_residual_ex.restype = ctypes.c_int
    L.oracle_append_residual_ex.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, P]
    L.oracle_append_projection.restype = ctypes.c_int
    L.oracle_append_projection.argtypes = [ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int, P]
    L.oracle_encode_tokens.restype = ctypes.c_int
    L.oracle_encode_tokens.argtypes = [ctypes.c_int, ctypes.c_int, P, ctypes.c_int64, P, P, P, P, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P, P, ctypes.c_int]
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
    sh.coef_bits = _coef_bits(cfg)
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
        _p(_u16(basisK)), _p(_u16(basisV)), _p(_coef(c["coefK"])), _p(_coef(c["coefV"])),
        _p(c["idxK"]), _p(c["idxV"]), _p(c["valK"]), _p(c["valV"]),
        _p(_u16(c["scaleK"])), _p(_u16(c["scaleV"])), *_cscales(c), _p(_u16(q)), float(alpha), _p(out),
        pa, npairs, int(threads))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return out


def _coef_bits(cfg) -> int:
    return int(getattr(cfg, "coef_bits", 16) or 16)


def _coef(a: np.ndarray) -> np.ndarray:
    """Coefficient array as the oracle reads it: fp16 bits, or int8 codes."""
    a = np.ascontiguousarray(a)
    return a if a.dtype == np.int8 else _u16(a)


def _cscales(c):
    """Pointers to the per-token coefficient block scales (8-bit form), or
    NULL for fp16 coefficients."""
    if "cscaleK" in c:
        return _p(_u16(c["cscaleK"])), _p(_u16(c["cscaleV"]))
    return None, None


def _shape(cfg, lay, tier_resid=None):
    B, Hkv, n_max, R = lay["coefK"].shape
    sh = _Shape()
    sh.batch, sh.num_kv_heads, sh.head_dim = B, Hkv, cfg.head_dim
    sh.num_q_heads = cfg.num_q_heads
    sh.r_max, sh.s_max, sh.n_max = R, lay["idxK"].shape[3], n_max
    sh.num_tiers = cfg.num_tiers
    sh.coef_bits = _coef_bits(cfg)
    res = tuple(tier_resid) if tier_resid is not None else cfg.resid_per_tier
    for k in range(cfg.num_tiers):
        sh.tier_rank[k] = cfg.tier_rank[k]
        sh.tier_resid[k] = res[k]
    return sh


def materialize(cfg, lay: Dict[str, np.ndarray], basisK: np.ndarray, basisV: np.ndarray,
                threads: int = 0):
    """(K^, V^) fp64 [B][H_kv][n_max][d]: Eq. (1) for every cached token in
    position order, zero past each sequence's length."""
    B, Hkv, n_max, R = lay["coefK"].shape
    d = cfg.head_dim
    sh = _shape(cfg, lay)
    K = np.zeros((B, Hkv, n_max, d), np.float64)
    V = np.zeros((B, Hkv, n_max, d), np.float64)
    c = {k: np.ascontiguousarray(v) for k, v in lay.items()}
    rc = lib().oracle_materialize(
        ctypes.byref(sh), _p(np.ascontiguousarray(c["n_tokens"], np.int64)), _p(c["tier"]),
        _p(_u16(basisK)), _p(_u16(basisV)), _p(_coef(c["coefK"])), _p(_coef(c["coefV"])),
        _p(c["idxK"]), _p(c["idxV"]), _p(c["valK"]), _p(c["valV"]),
        _p(_u16(c["scaleK"])), _p(_u16(c["scaleV"])), *_cscales(c), _p(K), _p(V), int(threads))
    if rc != 0:
        raise ValueError("oracle_materialize rejected its arguments")
    return K, V


def dense_decode(K: np.ndarray, V: np.ndarray, n_tokens, q: np.ndarray, alpha: Optional[float] = None,
                 threads: int = 0) -> np.ndarray:
    """Textbook attention [B][H_q][d] (fp64) over dense fp16 K, V
    [B][H_kv][n_max][d] (token rows) for q fp16 [B][H_q][d]."""
    B, Hkv, n_max, d = K.shape
    Hq = q.shape[1]
    if alpha is None:
        alpha = 1.0 / np.sqrt(d)
    out = np.zeros((B, Hq, d), np.float64)
    n = np.ascontiguousarray(np.asarray(n_tokens, np.int64).reshape(B))
    rc = lib().oracle_dense_decode(B, Hq, Hkv, d, n_max, _p(n), _p(_u16(np.ascontiguousarray(K))),
                                   _p(_u16(np.ascontiguousarray(V))), _p(_u16(np.ascontiguousarray(q))),
                                   float(alpha), _p(out), int(threads))
    if rc != 0:
        raise ValueError("oracle_dense_decode rejected its arguments")
    return out


# ------------------------------------------------------------------ probe (Eq. (3))
def probe_error(cfg, lay: Dict[str, np.ndarray], basisK: np.ndarray, basisV: np.ndarray,
                K_ref: np.ndarray, V_ref: np.ndarray, n_ref, qs: Sequence[np.ndarray],
                eps: float = 1e-6, alpha: Optional[float] = None) -> np.ndarray:
    """The paper's Eq. (3) (§3 Method, attention-output probes) per (sequence,
    KV head): || Attn(Q, K, V) - Attn(Q, K^, V^) ||_2 / (|| Attn(Q, K, V) ||_2 + eps),
    where K, V is the higher-fidelity dense fp16 cache (K_ref, V_ref
    [B][H_kv][n_max][d] token rows, n_ref tokens per sequence), K^, V^ the
    compressed cache (lay), and Q the recent query vectors qs (each fp16
    [B][H_q][d]) of the KV head's query heads; the norms run over every
    query position, query head and channel.  Returns fp64 [B][H_kv]."""
    B, Hkv = lay["coefK"].shape[:2]
    gq = cfg.num_q_heads // Hkv
    num = np.zeros((B, Hkv))
    den = np.zeros((B, Hkv))
    for q in qs:
        oc = decode(cfg, lay, basisK, basisV, q, alpha=alpha)
        oe = dense_decode(K_ref, V_ref, n_ref, q, alpha=alpha)
        dd = ((oe - oc) ** 2).reshape(B, Hkv, gq, -1).sum(axis=(2, 3))
        ee = (oe ** 2).reshape(B, Hkv, gq, -1).sum(axis=(2, 3))
        num += dd
        den += ee
    return np.sqrt(num) / (np.sqrt(den) + eps)


def probe_controller(tau: float, below: int, err: float, tol: float, step: float, patience: int,
                     tau_min: float, tau_max: float):
    """One probe interval of a depth window's router threshold (§3, the
    paragraph after Eq. (3)): an error above the window's tolerance lowers
    tau_m, so more of the window's tokens take higher residual rank; errors
    below it for `patience` probe intervals in a row raise tau_m, reducing
    residual storage.  tau moves by `step` in fp32 and stays in [tau_min,
    tau_max].  Returns (tau, below-tolerance run length)."""
    t = np.float32(tau)
    if err > tol:
        t = np.float32(t - np.float32(step))
        below = 0
    else:
        below += 1
        if below >= patience:
            t = np.float32(t + np.float32(step))
            below = 0
    t = np.float32(min(max(t, np.float32(tau_min)), np.float32(tau_max)))
    return float(t), below


# ------------------------------------------------------------------ append
def append_vector(basis: np.ndarray, x: np.ndarray, r: int, s: int, qmax: int,
                  gate: Optional[np.float16] = None, coef_bits: int = 16):
    """Encode one fp16 vector.  basis: fp16 [r_max][d]; x: fp16 [d].
    Returns (c, idx uint8[s], val int8[s], scale fp16) with c fp16[r]; with
    coef_bits 8, (c int8[r], idx, val, scale, coefficient block scale fp16)."""
    b = _u16(basis)
    xv = _u16(x)
    r_max, d = b.shape
    c = np.zeros(max(r, 1), np.uint16 if coef_bits == 16 else np.int8)
    idx = np.zeros(max(s, 1), np.uint8)
    val = np.zeros(max(s, 1), np.int8)
    sc = np.zeros(1, np.uint16)
    cs = np.zeros(1, np.uint16)
    g = 0x3C00 if gate is None else int(np.asarray(gate, np.float16).view(np.uint16))
    rc = lib().oracle_append_ex(d, r_max, _p(b), _p(xv), r, s, qmax, g, coef_bits, _p(c), _p(cs), _p(idx),
                                _p(val), _p(sc))
    if rc != 0:
        raise ValueError("oracle_append rejected its arguments")
    if coef_bits == 8:
        return c[:r], idx[:s], val[:s], sc.view(np.float16)[0], cs.view(np.float16)[0]
    return c[:r].view(np.float16), idx[:s], val[:s], sc.view(np.float16)[0]


def append_residual(basis: np.ndarray, x: np.ndarray, r: int, coef_bits: int = 16) -> np.ndarray:
    """fp32 residual e = x - B^T c of the encoder (step 2), c the stored
    coefficients (fp16, or int8 codes times their block scale)."""
    b = _u16(basis)
    xv = _u16(x)
    r_max, d = b.shape
    e = np.zeros(d, np.float32)
    if lib().oracle_append_residual_ex(d, r_max, _p(b), _p(xv), r, coef_bits, _p(e)) != 0:
        raise ValueError("oracle_append_residual rejected its arguments")
    return e


def append_projection(basis: np.ndarray, x: np.ndarray, r: int) -> np.ndarray:
    """fp32 sums of the encoder's step 1 (the coefficients before their fp16
    rounding), fp32 [r]."""
    b = _u16(basis)
    xv = _u16(x)
    r_max, d = b.shape
    out = np.zeros(max(r, 1), np.float32)
    if lib().oracle_append_projection(d, r_max, _p(b), _p(xv), r, _p(out)) != 0:
        raise ValueError("oracle_append_projection rejected its arguments")
    return out[:r]


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
    cb = _coef_bits(cfg)
    out = {}
    for z, x, bas, gate in (("K", k, basisK, gateK), ("V", v, basisV, gateV)):
        coef = np.zeros((B, H, R), np.float16 if cb == 16 else np.int8)
        cscale = np.zeros((B, H), np.float16)
        idx = np.zeros((B, H, S), np.uint8)
        val = np.zeros((B, H, S), np.int8)
        sc = np.zeros((B, H), np.float16)
        for b in range(B):
            for h in range(H):
                t = int(tier[b, h])
                r, s = cfg.tier_rank[t], res[t]
                g = None if gate is None else gate[b, h]
                enc = append_vector(bas[h], x[b, h], r, s, cfg.qmax, g, coef_bits=cb)
                coef[b, h, :r] = enc[0]
                idx[b, h, :s] = enc[1]
                val[b, h, :s] = enc[2]
                sc[b, h] = enc[3]
                if cb == 8:
                    cscale[b, h] = enc[4]
        out["coef" + z], out["idx" + z], out["val" + z], out["scale" + z] = coef, idx, val, sc
        if cb == 8:
            out["cscale" + z] = cscale
    return out


# ------------------------------------------------------------------ prefill
from .prefill import orth, prefill_bases, prefill_encode, range_finder, window_gram  # noqa: E402,F401
