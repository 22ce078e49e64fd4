"""Prefill compression -- TEST INFRASTRUCTURE (part of the CPU oracle).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module; the product never does.  Plain fp64 NumPy, one step per
statement, no blocking or reordering beyond what the steps below state.

What it computes (DepthWeave-KV paper, arXiv 2607.06523, §3 Method):

  * The shared bases are initialised after prefill from a small randomized
    low-rank sketch of the cached keys and values, independently per KV head
    and separately for K and V, over the layers of a depth window (second
    paragraph of §3).  The pages name no algorithm beyond "randomized
    low-rank sketch"; the plainest reading is the randomized range finder
    with subspace (power) iteration and a Rayleigh-Ritz step of Halko,
    Martinsson and Tropp ("Finding structure with randomness", SIAM Review
    2011, §4.5 and §5.3).  It is applied to the window's Gram matrix
    C = sum x x^T over every cached vector x of the window (all its layers,
    all sequences of the batch, every prefill token), whose dominant
    eigenvectors span the same subspace as the vectors' dominant right
    singular vectors:

        1. Y = C Omega               (Omega: a d x k Gaussian sketch, an input)
        2. Q = orth(Y)
        3. q times: Q = orth(C Q)    (power iterations)
        4. T = Q^T C Q,  T = U diag(theta) U^T   (Rayleigh-Ritz)
        5. Ritz vectors Q U in decreasing theta (ties: smaller index first),
           each with its largest-magnitude component made positive (first such
           component on ties)
        6. the basis: the first r_max Ritz vectors as rows, rounded to fp16.

    orth() is classical Gram-Schmidt applied twice per column over the
    columns of [Y | I_d] in order, skipping a column whose norm after the two
    passes is at most 2^-40 of its norm before them, until k columns are
    kept: for a full-rank Y it spans Y's columns (the QR factor up to column
    signs); for a rank-deficient Y it completes the basis with the first
    standard directions that are independent of the kept ones.

  * Then every prefill token is encoded exactly as an append would encode it
    (the data-path paragraph of §3 with Fig. 2: project onto the basis, keep
    the routed residual channels, quantise), in position order, with the
    router's per-token tier and gate as inputs.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

DEP_TOL = 2.0 ** -40


def window_gram(xs: Sequence[np.ndarray]) -> np.ndarray:
    """C = sum over the given vector sets of X^T X, in fp64.  xs: arrays of
    shape [n_i][d] (fp16 values are exact in fp64)."""
    d = xs[0].shape[-1]
    C = np.zeros((d, d), np.float64)
    for X in xs:
        X64 = np.asarray(X, np.float64).reshape(-1, d)
        C += X64.T @ X64
    return C


def orth(Y: np.ndarray) -> np.ndarray:
    """k orthonormal columns spanning Y [d][k] (see the module docstring)."""
    d, k = Y.shape
    cand = np.concatenate([Y, np.eye(d)], axis=1)
    Q = np.zeros((d, k), np.float64)
    kept = 0
    for c in range(cand.shape[1]):
        if kept == k:
            break
        v = cand[:, c].copy()
        n0 = np.sqrt(v @ v)
        for _ in range(2):
            if kept:
                v = v - Q[:, :kept] @ (Q[:, :kept].T @ v)
        n1 = np.sqrt(v @ v)
        if n0 == 0.0 or n1 <= DEP_TOL * n0:
            continue
        Q[:, kept] = v / n1
        kept += 1
    assert kept == k
    return Q


def sign_fix(V: np.ndarray) -> np.ndarray:
    """Each column with its first largest-magnitude component positive."""
    V = V.copy()
    for j in range(V.shape[1]):
        p = int(np.argmax(np.abs(V[:, j])))
        if V[p, j] < 0:
            V[:, j] = -V[:, j]
    return V


def range_finder(C: np.ndarray, omega: np.ndarray, r: int, q: int):
    """Basis of rank r from the Gram matrix C [d][d] and the sketch omega
    [d][k] with q power iterations.  Returns (B fp64 [r][d], theta fp64 [k]
    in decreasing order, B16 fp16 [r][d])."""
    d, k = omega.shape
    if not (0 < r <= k <= d):
        raise ValueError("need 0 < r <= k <= d")
    Y = C @ np.asarray(omega, np.float64)                    # 1.
    Q = orth(Y)                                              # 2.
    for _ in range(q):                                       # 3.
        Q = orth(C @ Q)
    T = Q.T @ (C @ Q)                                        # 4.
    T = 0.5 * (T + T.T)
    theta, U = np.linalg.eigh(T)
    order = np.argsort(-theta, kind="stable")                # 5.
    V = sign_fix(Q @ U[:, order])
    B = V[:, :r].T.copy()                                    # 6.
    return B, theta[order], B.astype(np.float16)


def window_vectors(K: np.ndarray, n_tokens, h: int):
    """The vectors of KV head h in one layer's prefill K (or V) [B][H][n][d]:
    each sequence's first n_b tokens."""
    return [K[b, h, : int(n_tokens[b])] for b in range(K.shape[0])]


def prefill_bases(cfg, K_layers: Sequence[np.ndarray], V_layers: Sequence[np.ndarray], n_tokens,
                  omega: np.ndarray, q: int = 2) -> Dict[str, np.ndarray]:
    """Bases of one depth window from the prefill keys and values of its
    layers.  K_layers, V_layers: fp16 [B][H][n_cap][d] per layer of the
    window; n_tokens [B]; omega: [2][H][d][k] (Z = K, V).  Returns
    {'K','V'}: fp16 [H][r_max][d]; {'K64','V64'}: the fp64 bases before
    rounding; {'thetaK','thetaV'}: fp64 [H][k] Ritz values; {'gramK',
    'gramV'}: fp64 [H][d][d]."""
    H, d, R = cfg.num_kv_heads, cfg.head_dim, cfg.r_max
    out = {}
    for zi, (z, layers) in enumerate((("K", K_layers), ("V", V_layers))):
        k = omega.shape[-1]
        b16 = np.zeros((H, R, d), np.float16)
        b64 = np.zeros((H, R, d), np.float64)
        th = np.zeros((H, k), np.float64)
        gram = np.zeros((H, d, d), np.float64)
        for h in range(H):
            xs = [x for L in layers for x in window_vectors(L, n_tokens, h)]
            C = window_gram(xs)
            b64[h], th[h], b16[h] = range_finder(C, omega[zi, h], R, q)
            gram[h] = C
        out[z], out[z + "64"], out["theta" + z], out["gram" + z] = b16, b64, th, gram
    return out


def prefill_encode(cfg, basisK: np.ndarray, basisV: np.ndarray, K: np.ndarray, V: np.ndarray, n_tokens,
                   tier: np.ndarray, gateK: Optional[np.ndarray] = None, gateV: Optional[np.ndarray] = None,
                   nthreads: int = 0) -> Dict[str, np.ndarray]:
    """Encodes one layer's prefill tokens into the logical cache (the token
    arrays of the seeded generator's layers, in position order).

    basisK, basisV: fp16 [H][r_max][d] (the window's bases); K, V: fp16
    [B][H][n_cap][d]; n_tokens [B]; tier: uint8 [B][H][n_cap]; gateK, gateV:
    optional fp16 [B][H][n_cap] (None: a gate of 1)."""
    from . import _coef_bits, _p, _u16, lib, max_threads
    B, H, _, d = K.shape
    n = int(np.max(n_tokens)) if len(n_tokens) else 0
    R, S = cfg.r_max, cfg.s_max
    cb = _coef_bits(cfg)
    ranks = np.asarray(cfg.tier_rank, np.int32)
    res = np.asarray(cfg.resid_per_tier, np.int32)
    lay = {"n_tokens": np.asarray(n_tokens, np.int64).copy(), "tier": np.zeros((B, H, n), np.uint8)}
    for z, X, bas, gate in (("K", K, basisK, gateK), ("V", V, basisV, gateV)):
        coef = np.zeros((B, H, n, R), np.float16 if cb == 16 else np.int8)
        cs = np.zeros((B, H, n), np.uint16)
        idx = np.zeros((B, H, n, max(S, 1)), np.uint8)
        val = np.zeros((B, H, n, max(S, 1)), np.int8)
        sc = np.zeros((B, H, n), np.uint16)
        for b in range(B):
            nb = int(n_tokens[b])
            for h in range(H):
                t = np.ascontiguousarray(tier[b, h, :nb]).astype(np.int64)
                if nb and t.max() >= cfg.num_tiers:
                    raise ValueError("tier out of range")
                lay["tier"][b, h, :nb] = t
                x = _u16(np.ascontiguousarray(X[b, h, :nb]))
                g = None if gate is None else _u16(np.ascontiguousarray(gate[b, h, :nb]))
                c_b = np.zeros((nb, R), coef.dtype)
                cs_b = np.zeros(nb, np.uint16)
                i_b = np.zeros((nb, max(S, 1)), np.uint8)
                v_b = np.zeros((nb, max(S, 1)), np.int8)
                s_b = np.zeros(nb, np.uint16)
                rc = lib().oracle_encode_tokens(
                    d, R, _p(_u16(np.ascontiguousarray(bas[h]))), nb, _p(x),
                    _p(np.ascontiguousarray(ranks[t])), _p(np.ascontiguousarray(res[t])),
                    None if g is None else _p(g), cfg.qmax, cb, R, max(S, 1), _p(c_b), _p(cs_b), _p(i_b),
                    _p(v_b), _p(s_b), nthreads or max_threads())
                if rc != 0:
                    raise ValueError("oracle_encode_tokens rejected its arguments")
                coef[b, h, :nb], cs[b, h, :nb] = c_b, cs_b
                idx[b, h, :nb], val[b, h, :nb], sc[b, h, :nb] = i_b, v_b, s_b
        lay["coef" + z] = coef
        lay["idx" + z] = idx[..., :S]
        lay["val" + z] = val[..., :S]
        lay["scale" + z] = sc.view(np.float16)
        if cb == 8:
            lay["cscale" + z] = cs.view(np.float16)
    return lay
