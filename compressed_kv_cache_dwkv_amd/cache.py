"""Device-memory plumbing around one libdwkv cache: torch owns the arena and
the decode workspaces; every operation is a call into libdwkv."""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import torch

from . import (dwkv_append, dwkv_arena_bytes, dwkv_check_errors, dwkv_clear_errors, dwkv_create,
               dwkv_decode_attn, dwkv_decode_splits, dwkv_decode_step, dwkv_destroy, dwkv_export_layer, dwkv_import_layer,
               dwkv_get_basis, dwkv_prefill_bases, dwkv_prefill_encode, dwkv_prefill_gram,
               dwkv_prefill_workspace_bytes, dwkv_read_counts, dwkv_reset, dwkv_set_basis, dwkv_workspace_bytes,
               make_config)


class CompressedKVCache:
    """One compressed cache (all layers) on one GPU.

    tier_capacity: token slots per (layer, sequence, KV head) for each tier;
    max_tokens: positions per (layer, sequence, KV head)."""

    def __init__(self, num_layers: int, layers_per_group: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, r_max: int, tier_rank: Sequence[int], tier_resid: Sequence[int],
                 resid_bits: int, max_batch: int, tier_capacity: Sequence[int], max_tokens: int,
                 decode_splits: int = 0, device: str = "cuda", coef_bits: int = 16):
        self.cfg = make_config(num_layers, layers_per_group, num_q_heads, num_kv_heads, head_dim,
                               r_max, tier_rank, tier_resid, resid_bits, max_batch, tier_capacity,
                               max_tokens, decode_splits, coef_bits)
        self.coef_bits = coef_bits
        self.device = torch.device(device)
        self.num_layers, self.num_q_heads, self.num_kv_heads = num_layers, num_q_heads, num_kv_heads
        self.head_dim, self.r_max, self.num_tiers = head_dim, r_max, len(tier_rank)
        self.s_max = max(tier_resid) if len(tier_resid) else 0
        self.max_batch = max_batch
        self.arena = torch.empty(dwkv_arena_bytes(self.cfg), dtype=torch.uint8, device=self.device)
        self.handle = dwkv_create(self.cfg, self.arena)
        self._ws: Dict[int, torch.Tensor] = {}
        self._pws: Optional[torch.Tensor] = None
        dwkv_reset(self.handle)

    # ------------------------------------------------------------------ setup
    @property
    def splits(self) -> int:
        """Decode workgroups per (sequence, KV head)."""
        return dwkv_decode_splits(self.handle)

    def workspace(self, batch: int) -> torch.Tensor:
        ws = self._ws.get(batch)
        if ws is None:
            ws = torch.zeros(dwkv_workspace_bytes(self.cfg, batch), dtype=torch.uint8, device=self.device)
            self._ws[batch] = ws
        return ws

    def set_basis(self, group: int, basisK: torch.Tensor, basisV: torch.Tensor) -> None:
        dwkv_set_basis(self.handle, group, basisK, basisV)

    def import_layer(self, layer: int, lay: Dict[str, torch.Tensor], n_tokens: Sequence[int]) -> None:
        dwkv_import_layer(self.handle, layer, lay, n_tokens)

    def export_layer(self, layer: int, batch: int, n_max: int):
        B, H, R, S = batch, self.num_kv_heads, self.r_max, max(self.s_max, 1)
        dev = self.device
        dst = {"tier": torch.zeros((B, H, n_max), dtype=torch.uint8, device=dev)}
        for z in "KV":
            dst["coef" + z] = torch.zeros((B, H, n_max, R), dtype=torch.float16 if self.coef_bits == 16 else torch.int8,
                                          device=dev)
            if self.coef_bits == 8:
                dst["cscale" + z] = torch.zeros((B, H, n_max), dtype=torch.float16, device=dev)
            dst["idx" + z] = torch.zeros((B, H, n_max, S), dtype=torch.uint8, device=dev)
            dst["val" + z] = torch.zeros((B, H, n_max, S), dtype=torch.int8, device=dev)
            dst["scale" + z] = torch.zeros((B, H, n_max), dtype=torch.float16, device=dev)
        counts = torch.zeros((B, H, self.num_tiers), dtype=torch.int32, device=dev)
        slots = torch.zeros((B, H, n_max), dtype=torch.int32, device=dev)
        dwkv_export_layer(self.handle, layer, dst, counts, slots)
        return dst, counts, slots

    def get_basis(self, group: int):
        """The window's bases (basisK, basisV), fp16 [H_kv][r_max][d] GPU tensors."""
        bk = torch.empty((self.num_kv_heads, self.r_max, self.head_dim), dtype=torch.float16, device=self.device)
        bv = torch.empty_like(bk)
        dwkv_get_basis(self.handle, group, bk, bv)
        return bk, bv

    # ------------------------------------------------------------------ prefill
    def prefill_workspace(self) -> torch.Tensor:
        if self._pws is None:
            self._pws = torch.zeros(dwkv_prefill_workspace_bytes(self.cfg), dtype=torch.uint8, device=self.device)
        return self._pws

    def prefill_gram(self, layer: int, k: torch.Tensor, v: torch.Tensor, n_tokens: torch.Tensor, first: bool) -> None:
        dwkv_prefill_gram(self.handle, layer, k, v, n_tokens, self.prefill_workspace(), first)

    def prefill_bases(self, group0: int, omega: torch.Tensor, power_iters: int = 2,
                      ritz: Optional[torch.Tensor] = None) -> None:
        if omega.dim() != 5 or tuple(omega.shape[1:4]) != (2, self.num_kv_heads, self.head_dim):
            raise ValueError("omega must be [n_groups][2][H_kv][head_dim][k]")
        dwkv_prefill_bases(self.handle, group0, omega, self.prefill_workspace(), power_iters, ritz)

    def prefill_encode(self, layer: int, k: torch.Tensor, v: torch.Tensor, n_tokens: torch.Tensor,
                       tier: torch.Tensor, gateK: Optional[torch.Tensor] = None,
                       gateV: Optional[torch.Tensor] = None) -> None:
        dwkv_prefill_encode(self.handle, layer, k, v, n_tokens, tier, self.prefill_workspace(), gateK, gateV)

    def gram(self, group: int) -> torch.Tensor:
        """The window's accumulated Gram sums, fp64 [2][H_kv][d][d] (a view of the workspace)."""
        H, d = self.num_kv_heads, self.head_dim
        n = 2 * H * d * d
        return self.prefill_workspace()[: (group + 1) * n * 8].view(torch.float64)[group * n:].view(2, H, d, d)

    def read_counts(self, layer: int, batch: int):
        return dwkv_read_counts(self.handle, layer, batch, self.num_kv_heads, self.num_tiers)

    # ------------------------------------------------------------------ hot path
    def decode(self, layer: int, q: torch.Tensor, out: Optional[torch.Tensor] = None,
               softmax_scale: Optional[float] = None) -> torch.Tensor:
        B = q.shape[0]
        if out is None:
            out = torch.empty((B, self.num_q_heads, self.head_dim), dtype=torch.float32, device=self.device)
        dwkv_decode_attn(self.handle, layer, q, out, self.workspace(B),
                         softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(self.head_dim))
        return out

    def append(self, layer: int, k: torch.Tensor, v: torch.Tensor, tier: torch.Tensor,
               gateK: Optional[torch.Tensor] = None, gateV: Optional[torch.Tensor] = None) -> None:
        dwkv_append(self.handle, layer, k, v, tier, gateK, gateV)

    def decode_step(self, layer: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    tier: torch.Tensor, gateK: Optional[torch.Tensor] = None,
                    gateV: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    softmax_scale: Optional[float] = None) -> torch.Tensor:
        """decode(q) over the cache as it stands, then append(k, v, tier), in one launch."""
        B = q.shape[0]
        if out is None:
            out = torch.empty((B, self.num_q_heads, self.head_dim), dtype=torch.float32, device=self.device)
        dwkv_decode_step(self.handle, layer, q, out, self.workspace(B), k, v, tier, gateK, gateV,
                         softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(self.head_dim))
        return out

    # ------------------------------------------------------------------ errors
    def check_errors(self) -> int:
        return dwkv_check_errors(self.handle)

    def clear_errors(self) -> None:
        dwkv_clear_errors(self.handle)

    def close(self) -> None:
        if self.handle is not None:
            dwkv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
