"""Workload shapes: five synthetic decode workloads.

Shapes stand in for the paper's long-context settings (64K-token prefill with
greedy decoding in the DepthWeave-KV paper, §4 Experiments; needle lengths
16K-128K in the same section).  No dataset item is reproduced: every value is
drawn from the seeded distributions below.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    num_layers: int
    layers_per_group: int          # G: layers sharing one basis (depth window)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int                  # d
    r_max: int                     # basis width
    tier_rank: Tuple[int, ...]     # coefficient rank per tier, ascending
    tier_prob: Tuple[float, ...]   # categorical mix of tiers
    resid_channels: int            # s: residual channels kept per token
    resid_bits: int                # 4 or 8
    n_tokens: int                  # context length already in the cache
    seed: int
    # router skew: positions < skew_prefix and round(skew_frac*n) random
    # positions are forced to the top tier (the 32K x 16 workload)
    skew_prefix: int = 0
    skew_frac: float = 0.0
    bench_steps: int = 1
    tier_resid: Tuple[int, ...] = field(default=())   # per-tier s; () = all s
    coef_bits: int = 16            # 16: fp16 coefficients; 8: int8 codes with a per-token fp16 block scale

    @property
    def group_q(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_groups(self) -> int:
        return (self.num_layers + self.layers_per_group - 1) // self.layers_per_group

    @property
    def num_tiers(self) -> int:
        return len(self.tier_rank)

    @property
    def qmax(self) -> int:
        return 7 if self.resid_bits == 4 else 127

    @property
    def resid_per_tier(self) -> Tuple[int, ...]:
        if self.tier_resid:
            return tuple(self.tier_resid)
        return tuple(self.resid_channels for _ in self.tier_rank)

    @property
    def s_max(self) -> int:
        return max(self.resid_per_tier) if self.tier_rank else 0

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


_LLAMA8B = dict(
    batch=1, num_layers=32, layers_per_group=4, num_q_heads=32, num_kv_heads=8,
    head_dim=128, r_max=64, tier_rank=(8, 16, 32, 64), tier_prob=(0.55, 0.25, 0.12, 0.08),
    resid_channels=8, resid_bits=4,
)

CONFIGS = (
    Config(name="tiny-ref-1k", batch=1, num_layers=2, layers_per_group=2, num_q_heads=4,
           num_kv_heads=1, head_dim=64, r_max=32, tier_rank=(4, 8, 16, 32),
           tier_prob=(0.60, 0.25, 0.10, 0.05), resid_channels=4, resid_bits=8,
           n_tokens=1024, seed=1000, bench_steps=1),
    Config(name="llama3-8b-8k", n_tokens=8192, seed=1001, bench_steps=256, **_LLAMA8B),
    Config(name="llama3-8b-64k", n_tokens=65536, seed=1002, bench_steps=256, **_LLAMA8B),
    Config(name="llama3-8b-32k-b16", n_tokens=32768, seed=1003, bench_steps=64,
           skew_prefix=64, skew_frac=0.02, **dict(_LLAMA8B, batch=16)),
    Config(name="llama3-70b-128k", batch=1, num_layers=80, layers_per_group=4, num_q_heads=64,
           num_kv_heads=8, head_dim=128, r_max=64, tier_rank=(8, 16, 32, 64),
           tier_prob=(0.60, 0.22, 0.12, 0.06), resid_channels=8, resid_bits=4,
           n_tokens=131072, seed=1004, bench_steps=64),
)


def get_config(i: int) -> Config:
    return CONFIGS[i]


def dense_kv_bytes(num_layers: int, num_kv_heads: int, head_dim: int, n_tokens: int,
                   batch: int = 1, elem_bytes: int = 2) -> int:
    """Bytes of an uncompressed K+V cache: 2 (K and V) x layers x heads x dim x
    tokens x element size (the KV-size arithmetic of the zhichai.net summary,
    Ch. 1.3 'The Long-Context Nightmare')."""
    return 2 * num_layers * num_kv_heads * head_dim * n_tokens * batch * elem_bytes


def compressed_bytes_per_token(rank: int, s: int, bits: int, coef_bits: int = 16) -> float:
    """Algorithmic bytes one token occupies per (layer, KV head), K and V
    together: the coefficients at the routed rank (fp16, or int8 codes plus
    one fp16 block scale), and per Z a residual block of s uint8 channel
    indices, s packed values and one fp16 scale (no block at all for a tier
    that keeps no residual channel)."""
    block = 0 if s == 0 else s + s * bits / 8 + 2
    coef = 2 * rank if coef_bits == 16 else rank + 2
    return 2 * coef + 2 * block
