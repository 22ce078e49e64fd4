"""GPU-side test plumbing: NumPy logical layers to device tensors, a cache
sized for a workload, decode/export back to NumPy."""
from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np
import torch

from workload import Config
from workload.gen import max_tier_counts


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_dev(lay: Dict[str, np.ndarray]) -> Dict[str, torch.Tensor]:
    return {k: dev(v) for k, v in lay.items() if k != "n_tokens"}


def make_cache(cfg: Config, capacity=None, extra: int = 16, splits: int = 0,
               max_tokens: Optional[int] = None, n: Optional[int] = None, all_top: bool = False):
    from compressed_kv_cache_dwkv_amd.cache import CompressedKVCache
    n = cfg.n_tokens if n is None else n
    if capacity is None:
        capacity = [int(c) + extra for c in max_tier_counts(cfg, n, all_top=all_top)]
    return CompressedKVCache(
        cfg.num_layers, cfg.layers_per_group, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
        cfg.r_max, cfg.tier_rank, cfg.resid_per_tier, cfg.resid_bits, cfg.batch, capacity,
        max_tokens if max_tokens is not None else n + extra, splits, coef_bits=cfg.coef_bits)


def load_bases(cache, bases: Dict[str, np.ndarray], groups: Optional[Iterable[int]] = None):
    G = bases["K"].shape[0]
    for m in (range(G) if groups is None else groups):
        cache.set_basis(m, dev(bases["K"][m]), dev(bases["V"][m]))


def load_layer(cache, layer: int, lay: Dict[str, np.ndarray]):
    cache.import_layer(layer, to_dev(lay), [int(x) for x in lay["n_tokens"]])


def decode_np(cache, layer: int, q: np.ndarray, scale: Optional[float] = None) -> np.ndarray:
    out = cache.decode(layer, dev(q), softmax_scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def export_np(cache, layer: int, batch: int, n_max: int):
    dst, counts, slots = cache.export_layer(layer, batch, n_max)
    torch.cuda.synchronize()
    return ({k: v.cpu().numpy() for k, v in dst.items()}, counts.cpu().numpy(), slots.cpu().numpy())


def norm_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per (b, query head): max_j |got - ref| / max_j |ref| (row-max normalised)."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return num / den
