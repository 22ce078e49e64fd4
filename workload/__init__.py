"""Seeded synthetic inputs for the DepthWeave-KV decode path.

This module is the only code shared by the HIP path's tests/bench and by the
CPU oracle's tests.  It draws random numbers and lays them out; it holds none
of the method's arithmetic (no reconstruction, no projection, no attention, no
quantisation decisions).  Every array it returns is the *logical* cache of one
layer in token-position order -- the representation of Eq. (1) of the
DepthWeave-KV paper (arXiv 2607.06523, §3 Method):

    X^Z_{l,h,t} = A^Z_{l,h,t} B^Z_{m,h} + g R^Z_{l,h,t},   Z in {K, V}

with the coefficient vector A stored at the token's rank tier, and the sparse
quantised residual g R stored as (channel index, integer value, fp16 scale).

Value distributions follow the five workload configurations (tiny reference,
Llama-3-8B-shaped at 8K / 64K / 32Kx16, Llama-3-70B-shaped at 128K).
"""
from .configs import Config, CONFIGS, get_config, dense_kv_bytes, compressed_bytes_per_token
from .gen import (
    make_bases,
    gen_layer,
    gen_query,
    gen_append_inputs,
    layer_bases,
    empty_layer,
    gen_prefill,
    gen_sketch,
    gen_tiers,
    gen_gates,
)

__all__ = [
    "Config", "CONFIGS", "get_config", "dense_kv_bytes", "compressed_bytes_per_token",
    "make_bases", "gen_layer", "gen_query", "gen_append_inputs", "layer_bases", "empty_layer",
    "gen_prefill", "gen_sketch", "gen_tiers", "gen_gates",
]
