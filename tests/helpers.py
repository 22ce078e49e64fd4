"""Small shared helpers for the tests: tiny workload shapes, exact bases, and
textbook dense materialisation used as independent cross-checks."""
from __future__ import annotations

import numpy as np

from workload import Config


def tiny_config(**kw) -> Config:
    base = dict(name="tiny", batch=2, num_layers=2, layers_per_group=2, num_q_heads=4,
                num_kv_heads=2, head_dim=16, r_max=16, tier_rank=(4, 8, 16),
                tier_prob=(0.5, 0.3, 0.2), resid_channels=3, resid_bits=8, n_tokens=7, seed=4242)
    base.update(kw)
    return Config(**base)


def signed_permutation_basis(d: int, r_max: int, seed: int) -> tuple:
    """Basis whose vector i is sign_i * e_{perm_i}: exact in fp16 and exactly
    orthonormal.  Returns (fp16 [r_max][d], perm[r_max], sign[r_max])."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(d)[:r_max]
    sign = rng.choice([-1.0, 1.0], size=r_max)
    b = np.zeros((r_max, d), np.float16)
    b[np.arange(r_max), perm] = sign
    return b, perm, sign


def dense_from_logical(cfg: Config, lay: dict, basis: np.ndarray, z: str) -> np.ndarray:
    """Textbook materialisation [B][H][n][d] in fp64: coefficients times basis
    vectors (NumPy matmul) plus the sparse residual written into its channels."""
    coef = lay["coef" + z].astype(np.float64)                 # [B][H][n][R]
    if "cscale" + z in lay:                                   # 8-bit codes times their block scale
        coef = coef * lay["cscale" + z].astype(np.float64)[..., None]
    B, H, n, R = coef.shape
    bas = basis.astype(np.float64)                            # [H][R][d]
    x = np.einsum("bhnr,hrd->bhnd", coef, bas)
    res = tuple(cfg.resid_per_tier)
    scale = lay["scale" + z].astype(np.float64)
    for b in range(B):
        for h in range(H):
            for t in range(int(lay["n_tokens"][b])):
                s = res[int(lay["tier"][b, h, t])]
                for u in range(s):
                    x[b, h, t, int(lay["idx" + z][b, h, t, u])] += scale[b, h, t] * float(lay["val" + z][b, h, t, u])
    return x


def sdpa_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_tokens, scale: float) -> np.ndarray:
    """torch scaled_dot_product_attention in fp64 on CPU, one query per head,
    grouped-query heads (query head g reads KV head g // (H_q/H_kv))."""
    import torch
    import torch.nn.functional as F
    B, Hq, d = q.shape
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(n_tokens[b])
        if n == 0:
            continue
        qt = torch.from_numpy(q[b].astype(np.float64)).reshape(1, Hq, 1, d)
        kt = torch.from_numpy(np.ascontiguousarray(k[b, :, :n])).unsqueeze(0)
        vt = torch.from_numpy(np.ascontiguousarray(v[b, :, :n])).unsqueeze(0)
        o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
        out[b] = o.reshape(Hq, d).numpy()
    return out


def rel_err(a: np.ndarray, ref: np.ndarray) -> float:
    """max |a - ref| / max |ref| over the last axis, maximised over rows."""
    num = np.abs(a - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())


def extend_layer(lay: dict, enc: dict, tier: np.ndarray, n: int) -> dict:
    """The logical layer `lay` (n tokens per sequence) with the oracle's
    encoding `enc` of one appended token per (b, KV head) at position n."""
    out = {}
    for key, v in lay.items():
        if key == "n_tokens":
            out[key] = v + 1
            continue
        shape = list(v.shape)
        shape[2] += 1
        nv = np.zeros(shape, v.dtype)
        nv[:, :, :n] = v
        out[key] = nv
    out["tier"][:, :, n] = tier
    for z in "KV":
        out["coef" + z][:, :, n] = enc["coef" + z]
        out["idx" + z][:, :, n] = enc["idx" + z]
        out["val" + z][:, :, n] = enc["val" + z]
        out["scale" + z][:, :, n] = enc["scale" + z]
        if "cscale" + z in enc:
            out["cscale" + z][:, :, n] = enc["cscale" + z]
    return out
