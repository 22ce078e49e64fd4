"""Seeded generators (NumPy Philox, one sub-stream per (workload, field, index)).

Distributions (per workload configuration):
  * bases: per (depth group m, KV head h, Z) a d x r_max Gaussian matrix,
    orthonormalised by QR in fp64 with the sign fixed so diag(R) > 0, then
    rounded to fp16.  Stored as r_max rows of d values (basis vector i is
    row i).  The fp64 matrix is also returned (used only to synthesise new
    tokens for the append step).
  * rank tier per (b, m, h, t): categorical with the workload's mix; shared by
    the layers of a depth group and by K and V (Eq. (2) of the paper indexes
    the routed rank by window, head and token).  Optional router skew forces
    a prefix and a random 2% of positions to the top tier.
  * coefficients c_i ~ N(0, 1/(1+i)) (variance), i < r_tier, rounded to fp16;
    entries at i >= r_tier are zero (never stored by the cache).  In the
    8-bit blockwise form the codes and block scales are drawn directly:
    codes rint(N(0,1) * 127 / (3 sqrt(1+i))) clipped to [-127, 127], and a
    per-token scale fp16(3/127 * exp(0.1 N(0,1))), so that code * scale has
    about the fp16 form's variance.
  * residual: s distinct uniform channels (ascending), integer values uniform
    on [-qmax, qmax], scale = fp16(0.01 |N(0,1)|).
  * queries: fp16 N(0,1).
  * prefill keys and values (the input of the prefill compression): per
    (depth group m, KV head h, Z) a random orthogonal d x d matrix U (QR of a
    Gaussian, diag(R) > 0) and a geometric spectrum sigma_i = decay^i (decay
    0.93 for K, 0.96 for V); each layer of the group scales it by its own
    exp(0.1 N(0,1)) per channel, and token t is U (sigma_l * g_t) plus an
    isotropic N(0, noise^2) floor (noise 0.02), g_t ~ N(0, I), rounded to
    fp16.  Neighbouring layers thus share a dominant channel subspace with
    layer-specific deviations.  Positions at or beyond a sequence's length
    hold the `tail` value.
  * the range finder's Gaussian sketch: N(0,1) fp32 [d][k] per (m, Z, h).
  * prefill gates: per token fp16, 1.0 with probability 0.3, else uniform
    on [0.25, 1).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .configs import Config

_FIELDS = {
    "basis": 1, "tier": 2, "skewpos": 3, "coef": 4, "idx": 5, "val": 6, "scale": 7,
    "query": 8, "app_tier": 9, "app_coef": 10, "app_idx": 11, "app_val": 12,
    "app_scale": 13, "needle": 14, "cscale": 15, "pf_rot": 16, "pf_spec": 17, "pf_x": 18,
    "pf_noise": 19, "pf_omega": 20, "pf_gate": 21,
}


def _rng(seed: int, field: str, *key: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), _FIELDS[field]] + [int(k) for k in key])
    return np.random.Generator(np.random.Philox(ss))


def _seed_of(cfg: Config, variant_seed: int) -> int:
    return cfg.seed if variant_seed == 0 else cfg.seed * 7919 + variant_seed


# --------------------------------------------------------------------------- bases
def make_bases(cfg: Config, identity: bool = False, variant_seed: int = 0) -> Dict[str, np.ndarray]:
    """Shared channel bases for every depth group.

    Returns {'K','V'}: fp16 [num_groups][H_kv][r_max][d] and {'K64','V64'}: the
    fp64 orthonormal matrices before rounding, [num_groups][H_kv][d][r_max].
    identity=True gives B = I (needs r_max == d)."""
    seed = _seed_of(cfg, variant_seed)
    d, r = cfg.head_dim, cfg.r_max
    out = {}
    for zi, z in enumerate("KV"):
        b16 = np.zeros((cfg.num_groups, cfg.num_kv_heads, r, d), np.float16)
        b64 = np.zeros((cfg.num_groups, cfg.num_kv_heads, d, r), np.float64)
        for m in range(cfg.num_groups):
            for h in range(cfg.num_kv_heads):
                if identity:
                    if r != d:
                        raise ValueError("identity basis needs r_max == head_dim")
                    q = np.eye(d)
                else:
                    g = _rng(seed, "basis", zi, m, h).standard_normal((d, r))
                    q, rr = np.linalg.qr(g)
                    q = q * np.sign(np.diag(rr))[None, :]
                b64[m, h] = q
                b16[m, h] = q.T.astype(np.float16)
        out[z] = b16
        out[z + "64"] = b64
    return out


def layer_bases(bases: Dict[str, np.ndarray], cfg: Config, layer: int) -> Dict[str, np.ndarray]:
    m = layer // cfg.layers_per_group
    return {k: v[m] for k, v in bases.items()}


# --------------------------------------------------------------------------- tiers
def _tiers(cfg: Config, layer: int, n: int, seed: int, all_top: bool) -> np.ndarray:
    T = cfg.num_tiers
    m = layer // cfg.layers_per_group
    tier = np.empty((cfg.batch, cfg.num_kv_heads, n), np.uint8)
    if all_top:
        tier[:] = T - 1
        return tier
    probs = np.asarray(cfg.tier_prob, np.float64)
    cdf = np.cumsum(probs / probs.sum())
    for b in range(cfg.batch):
        u = _rng(seed, "tier", b, m).random((cfg.num_kv_heads, n))
        tier[b] = np.minimum(np.searchsorted(cdf, u, side="right"), T - 1).astype(np.uint8)
        if cfg.skew_prefix or cfg.skew_frac:
            tier[b, :, : min(cfg.skew_prefix, n)] = T - 1
            k = int(round(cfg.skew_frac * n))
            if k > 0:
                pos = _rng(seed, "skewpos", b).choice(n, size=k, replace=False)
                tier[b, :, pos] = T - 1
    return tier


def _distinct_sorted_channels(rng: np.random.Generator, rows: int, s: int, d: int) -> np.ndarray:
    """rows x s distinct channel indices in [0, d), ascending, by rejection."""
    idx = np.sort(rng.integers(0, d, size=(rows, s)), axis=1)
    while s > 1:
        bad = np.nonzero((np.diff(idx, axis=1) == 0).any(axis=1))[0]
        if bad.size == 0:
            break
        idx[bad] = np.sort(rng.integers(0, d, size=(bad.size, s)), axis=1)
    return idx.astype(np.uint8)


# --------------------------------------------------------------------------- layer
def empty_layer(cfg: Config, n: int = 0) -> Dict[str, np.ndarray]:
    B, H, R, S = cfg.batch, cfg.num_kv_heads, cfg.r_max, cfg.s_max
    lay = {
        "n_tokens": np.full((B,), n, np.int64),
        "tier": np.zeros((B, H, n), np.uint8),
    }
    for z in "KV":
        lay["coef" + z] = np.zeros((B, H, n, R), np.float16 if cfg.coef_bits == 16 else np.int8)
        if cfg.coef_bits == 8:
            lay["cscale" + z] = np.zeros((B, H, n), np.float16)
        lay["idx" + z] = np.zeros((B, H, n, S), np.uint8)
        lay["val" + z] = np.zeros((B, H, n, S), np.int8)
        lay["scale" + z] = np.zeros((B, H, n), np.float16)
    return lay


def gen_layer(cfg: Config, layer: int, n: Optional[int] = None, all_top: bool = False,
              variant_seed: int = 0) -> Dict[str, np.ndarray]:
    """Logical (position-ordered) compressed cache of one layer.

    Arrays: n_tokens[B] int64; tier[B][H_kv][n] uint8; coef{K,V}[B][H_kv][n][r_max]
    fp16 (zero at i >= rank); idx{K,V}[B][H_kv][n][s_max] uint8 ascending within
    the token's s_tier entries; val{K,V} int8 likewise; scale{K,V}[B][H_kv][n] fp16.
    Entries beyond a token's own s_tier are zero."""
    n = cfg.n_tokens if n is None else int(n)
    seed = _seed_of(cfg, variant_seed)
    lay = empty_layer(cfg, n)
    tier = _tiers(cfg, layer, n, seed, all_top)
    lay["tier"] = tier
    ranks = np.asarray(cfg.tier_rank)
    svec = np.asarray(cfg.resid_per_tier)
    d, qmax = cfg.head_dim, cfg.qmax
    std_all = np.sqrt(1.0 / (1.0 + np.arange(cfg.r_max)))
    for zi, z in enumerate("KV"):
        coef, idx, val, scale = lay["coef" + z], lay["idx" + z], lay["val" + z], lay["scale" + z]
        for b in range(cfg.batch):
            rc = _rng(seed, "coef", layer, zi, b)
            ri = _rng(seed, "idx", layer, zi, b)
            rv = _rng(seed, "val", layer, zi, b)
            rs = _rng(seed, "scale", layer, zi, b)
            for k in range(cfg.num_tiers):
                sel = np.nonzero(tier[b] == k)          # (head, pos) pairs, row-major
                cnt = sel[0].size
                if cnt == 0:
                    continue
                r = int(ranks[k])
                c = rc.standard_normal((cnt, r), dtype=np.float32) * std_all[:r].astype(np.float32)
                if cfg.coef_bits == 8:
                    codes = np.clip(np.rint(c * np.float32(127.0 / 3.0)), -127, 127).astype(np.int8)
                    coef[b][sel[0], sel[1], :r] = codes
                    u = _rng(seed, "cscale", layer, zi, b, k).standard_normal(cnt)
                    lay["cscale" + z][b][sel[0], sel[1]] = (3.0 / 127.0 * np.exp(0.1 * u)).astype(np.float16)
                else:
                    coef[b][sel[0], sel[1], :r] = c.astype(np.float16)
                s = int(svec[k])
                if s == 0:
                    continue
                idx[b][sel[0], sel[1], :s] = _distinct_sorted_channels(ri, cnt, s, d)
                val[b][sel[0], sel[1], :s] = rv.integers(-qmax, qmax + 1, size=(cnt, s)).astype(np.int8)
                scale[b][sel[0], sel[1]] = (0.01 * np.abs(rs.standard_normal(cnt))).astype(np.float16)
    return lay


# --------------------------------------------------------------------------- queries
def gen_query(cfg: Config, layer: int, step: int = 0, peak: float = 1.0,
              variant_seed: int = 0) -> np.ndarray:
    """fp16 [B][H_q][d] ~ N(0,1), times `peak` (16 gives a peaked softmax)."""
    seed = _seed_of(cfg, variant_seed)
    q = _rng(seed, "query", layer, step).standard_normal((cfg.batch, cfg.num_q_heads, cfg.head_dim))
    return (q * peak).astype(np.float16)


def gen_append_inputs(cfg: Config, layer: int, step: int, bases: Dict[str, np.ndarray],
                      variant_seed: int = 0) -> Dict[str, np.ndarray]:
    """A new token per (b, KV head) for the append step.

    The token is synthesised like a cache token at full rank (c_i ~ N(0,1/(1+i))
    on the fp64 orthonormal basis, plus an s-sparse residual) and rounded to
    fp16.  Its rank tier is drawn from the workload's mix, shared by the
    layers of a depth group.  Returns k, v: fp16 [B][H_kv][d]; tier: uint8
    [B][H_kv]."""
    seed = _seed_of(cfg, variant_seed)
    m = layer // cfg.layers_per_group
    B, H, d, R = cfg.batch, cfg.num_kv_heads, cfg.head_dim, cfg.r_max
    probs = np.asarray(cfg.tier_prob, np.float64)
    cdf = np.cumsum(probs / probs.sum())
    u = _rng(seed, "app_tier", m, step).random((B, H))
    tier = np.minimum(np.searchsorted(cdf, u, side="right"), cfg.num_tiers - 1).astype(np.uint8)
    out = {"tier": tier}
    std = np.sqrt(1.0 / (1.0 + np.arange(R)))
    s = cfg.resid_channels
    for zi, z in enumerate("KV"):
        b64 = bases[z + "64"][m]                   # [H][d][R]
        c = _rng(seed, "app_coef", layer, step, zi).standard_normal((B, H, R)) * std
        x = np.einsum("hdr,bhr->bhd", b64, c)
        if s > 0:
            idx = _distinct_sorted_channels(_rng(seed, "app_idx", layer, step, zi), B * H, s, d)
            val = _rng(seed, "app_val", layer, step, zi).integers(-cfg.qmax, cfg.qmax + 1, size=(B * H, s))
            sc = 0.01 * np.abs(_rng(seed, "app_scale", layer, step, zi).standard_normal(B * H))
            xf = x.reshape(B * H, d)
            np.add.at(xf, (np.repeat(np.arange(B * H), s), idx.reshape(-1).astype(np.int64)),
                      (sc[:, None] * val).reshape(-1))
            x = xf.reshape(B, H, d)
        out[z.lower()] = x.astype(np.float16)
    return out


def needle_positions(n: int, count: int = 3) -> Sequence[int]:
    """Start, middle and end positions of an n-token context."""
    if n <= 0:
        return []
    return sorted(set([0, n // 2, n - 1][:count]))


def plant_needles(cfg: Config, lay: Dict[str, np.ndarray], basisK16: np.ndarray, q: np.ndarray,
                  positions: Sequence[int], lead: float = 60.0) -> Dict[str, np.ndarray]:
    """Turn the tokens at `positions` of every (b, KV head) into needles for the
    first query head of the head's group: top tier, K coefficients along the
    query's projection onto the (fp16) basis, scaled so that query's logit is
    about `lead` (natural-log units, softmax scale 1/sqrt(d)) -- far above the
    O(1) logits of ordinary tokens.  Residuals of needles are zeroed.
    basisK16: [H_kv][r_max][d] fp16; q: [B][H_q][d] fp16.  Modifies `lay`."""
    top = cfg.num_tiers - 1
    r = cfg.tier_rank[top]
    alpha = 1.0 / np.sqrt(cfg.head_dim)
    for b in range(cfg.batch):
        for h in range(cfg.num_kv_heads):
            g0 = h * cfg.group_q
            proj = basisK16[h, :r].astype(np.float64) @ q[b, g0].astype(np.float64)
            lam = lead / (alpha * max(float(proj @ proj), 1e-6))
            for t in positions:
                lay["tier"][b, h, t] = top
                lay["coefK"][b, h, t, :] = 0
                if cfg.coef_bits == 8:
                    # the needle's coefficients as codes and a block scale
                    v = (lam * proj).astype(np.float32)
                    cs = (np.abs(v).max() / np.float32(127)).astype(np.float16)
                    lay["cscaleK"][b, h, t] = cs
                    lay["coefK"][b, h, t, :r] = np.clip(np.rint(v / np.float32(cs)), -127, 127).astype(np.int8)
                else:
                    lay["coefK"][b, h, t, :r] = (lam * proj).astype(np.float16)
                for z in "KV":
                    lay["idx" + z][b, h, t] = 0
                    lay["val" + z][b, h, t] = 0
                    lay["scale" + z][b, h, t] = 0
    return lay


def max_tier_counts(cfg: Config, n: Optional[int] = None, all_top: bool = False,
                    variant_seed: int = 0) -> np.ndarray:
    """Largest number of tokens any (layer, sequence, KV head) of the workload
    holds in each tier (used to size tier capacities)."""
    n = cfg.n_tokens if n is None else int(n)
    seed = _seed_of(cfg, variant_seed)
    mx = np.zeros(cfg.num_tiers, np.int64)
    for m in range(cfg.num_groups):
        tier = _tiers(cfg, m * cfg.layers_per_group, n, seed, all_top)
        for k in range(cfg.num_tiers):
            mx[k] = max(mx[k], int((tier == k).sum(axis=-1).max()) if n > 0 else 0)
    return mx


# --------------------------------------------------------------------------- prefill
def gen_prefill(cfg: Config, layer: int, n: Optional[int] = None, lengths: Optional[Sequence[int]] = None,
                tail: float = 0.0, noise: float = 0.02, variant_seed: int = 0):
    """Prefill keys and values of one layer: (K, V) fp16 [B][H_kv][n][d] with
    n = max(lengths) (default: every sequence cfg.n_tokens long)."""
    n = cfg.n_tokens if n is None else int(n)
    lengths = [n] * cfg.batch if lengths is None else [int(x) for x in lengths]
    n_cap = max(lengths) if lengths else 0
    seed = _seed_of(cfg, variant_seed)
    m = layer // cfg.layers_per_group
    d, H = cfg.head_dim, cfg.num_kv_heads
    out = []
    for zi, decay in enumerate((0.93, 0.96)):
        X = np.full((cfg.batch, H, n_cap, d), tail, np.float16)
        for h in range(H):
            g = _rng(seed, "pf_rot", m, zi, h).standard_normal((d, d))
            U, rr = np.linalg.qr(g)
            U = (U * np.sign(np.diag(rr))[None, :]).astype(np.float32)
            sig = decay ** np.arange(d) * np.exp(0.1 * _rng(seed, "pf_spec", m, zi, h, layer).standard_normal(d))
            A = (sig[:, None] * U.T).astype(np.float32)          # x = g @ A = U (sig * g)
            for b in range(cfg.batch):
                nb = lengths[b]
                if nb == 0:
                    continue
                gx = _rng(seed, "pf_x", layer, zi, b, h).standard_normal((nb, d), dtype=np.float32)
                e = _rng(seed, "pf_noise", layer, zi, b, h).standard_normal((nb, d), dtype=np.float32)
                X[b, h, :nb] = (gx @ A + np.float32(noise) * e).astype(np.float16)
        out.append(X)
    return out[0], out[1]


def gen_sketch(cfg: Config, k: int, variant_seed: int = 0) -> np.ndarray:
    """Gaussian sketches: fp32 [num_groups][2][H_kv][d][k]."""
    seed = _seed_of(cfg, variant_seed)
    om = np.zeros((cfg.num_groups, 2, cfg.num_kv_heads, cfg.head_dim, k), np.float32)
    for m in range(cfg.num_groups):
        for zi in range(2):
            for h in range(cfg.num_kv_heads):
                om[m, zi, h] = _rng(seed, "pf_omega", m, zi, h).standard_normal((cfg.head_dim, k), dtype=np.float32)
    return om


def gen_tiers(cfg: Config, layer: int, n: Optional[int] = None, variant_seed: int = 0) -> np.ndarray:
    """The router's tier per (b, KV head, position): uint8 [B][H_kv][n], shared
    by the layers of a depth group (the mix of the cached layers)."""
    n = cfg.n_tokens if n is None else int(n)
    return _tiers(cfg, layer, n, _seed_of(cfg, variant_seed), False)


def gen_gates(cfg: Config, layer: int, n: Optional[int] = None, variant_seed: int = 0):
    """Per-token residual gates (gateK, gateV): fp16 [B][H_kv][n]."""
    n = cfg.n_tokens if n is None else int(n)
    seed = _seed_of(cfg, variant_seed)
    out = []
    for zi in range(2):
        r = _rng(seed, "pf_gate", layer, zi)
        u = r.random((cfg.batch, cfg.num_kv_heads, n))
        g = 0.25 + 0.75 * r.random((cfg.batch, cfg.num_kv_heads, n))
        out.append(np.where(u < 0.3, 1.0, g).astype(np.float16))
    return out[0], out[1]
