"""Python binding of libdwkv (include/dwkv.h): DepthWeave-KV compressed-KV
decode attention and append on MI355X.

Argument marshalling only: every step runs in the HIP kernels of libdwkv.so.
The functions carry the C names; tensors are torch tensors on the GPU (the
binding passes their data pointers), streams default to torch's current
stream.  There is no CPU fallback: importing this package on a tree where
libdwkv.so has not been built raises ImportError.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Dict, Optional, Sequence

import numpy as np

# torch first: it loads the HIP runtime (libamdhip64.so.7) whose device memory
# and streams the callers hand over; libdwkv.so must bind to that same
# runtime instance rather than load a second copy from the ROCm install.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdwkv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dwkv.h")
MAX_TIERS = 8

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python compressed_kv_cache_dwkv_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

DWKV_OK = 0
DWKV_ERR_INVALID_ARG = -1
DWKV_ERR_UNSUPPORTED = -2
DWKV_ERR_WORKSPACE = -3
DWKV_ERR_CAPACITY = -4
DWKV_ERR_HIP = -5
DWKV_ERR_DEVICE = -6
DWKV_DEVERR_TIER_FULL = 1
DWKV_DEVERR_POS_FULL = 2
DWKV_DEVERR_BAD_TIER = 4
DWKV_DEVERR_BAD_INDEX = 8
DWKV_NOALLOC_SCRATCH_BYTES = 4 << 20
DWKV_NOALLOC_MAX_PAIRS = 1024


class dwkv_config(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("layers_per_group", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("r_max", ctypes.c_int32), ("num_tiers", ctypes.c_int32),
        ("tier_rank", ctypes.c_int32 * MAX_TIERS), ("tier_resid", ctypes.c_int32 * MAX_TIERS),
        ("resid_bits", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("decode_splits", ctypes.c_int32),
        ("tier_capacity", ctypes.c_int64 * MAX_TIERS), ("max_tokens", ctypes.c_int64),
        ("coef_bits", ctypes.c_int32),
    ]


class dwkv_logical_layer(ctypes.Structure):
    _fields_ = [
        ("n_max", ctypes.c_int64), ("tier", ctypes.c_void_p),
        ("coefK", ctypes.c_void_p), ("coefV", ctypes.c_void_p),
        ("idxK", ctypes.c_void_p), ("idxV", ctypes.c_void_p),
        ("valK", ctypes.c_void_p), ("valV", ctypes.c_void_p),
        ("scaleK", ctypes.c_void_p), ("scaleV", ctypes.c_void_p),
        ("cscaleK", ctypes.c_void_p), ("cscaleV", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SIGS = {
    "dwkv_arena_bytes": [ctypes.POINTER(dwkv_config), ctypes.POINTER(ctypes.c_size_t)],
    "dwkv_create": [ctypes.POINTER(dwkv_config), _P, ctypes.c_size_t, ctypes.POINTER(_P)],
    "dwkv_destroy": [_P],
    "dwkv_reset": [_P, _P],
    "dwkv_set_basis": [_P, _I, _P, _P, _P],
    "dwkv_get_basis": [_P, _I, _P, _P, _P],
    "dwkv_import_layer": [_P, _I, ctypes.POINTER(dwkv_logical_layer), ctypes.POINTER(ctypes.c_int64), _I, _P],
    "dwkv_export_layer": [_P, _I, ctypes.POINTER(dwkv_logical_layer), _P, _P, _I, _P],
    "dwkv_read_counts": [_P, _I, _I, _P, _P],
    "dwkv_workspace_bytes": [ctypes.POINTER(dwkv_config), _I, ctypes.POINTER(ctypes.c_size_t)],
    "dwkv_decode_splits": [_P, ctypes.POINTER(_I)],
    "dwkv_decode_attn": [_P, _I, _P, _I, ctypes.c_float, _P, _P, ctypes.c_size_t, _P],
    "dwkv_append": [_P, _I, _P, _P, _P, _P, _P, _I, _P],
    "dwkv_decode_step": [_P, _I, _P, _I, ctypes.c_float, _P, _P, ctypes.c_size_t, _P, _P, _P, _P, _P, _P],
    "dwkv_decode_step_noalloc": [_P, _I, _P, _I, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P],
    "dwkv_materialize_layer": [_P, _I, _I, _P, _P, ctypes.c_int64, _P, _P],
    "dwkv_dense_workspace_bytes": [_I, _I, _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
    "dwkv_dense_decode": [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_int64, _I, ctypes.c_float, _P, _P,
                          ctypes.c_size_t, _P],
    "dwkv_stream_probe": [_P, ctypes.c_int64, _I, _I, ctypes.c_uint32, _P, _P],
    "dwkv_probe_workspace_bytes": [ctypes.POINTER(dwkv_config), _I, _I, _I, ctypes.POINTER(ctypes.c_size_t)],
    "dwkv_probe_error": [_P, _I, _P, _I, _I, _P, _P, _P, ctypes.c_int64, _I, ctypes.c_float, ctypes.c_float, _P, _P,
                         ctypes.c_size_t, _P],
    "dwkv_probe_update": [_P, _P, _I, _P, ctypes.c_float, ctypes.c_float, _I, ctypes.c_float, ctypes.c_float],
    "dwkv_prefill_workspace_bytes": [ctypes.POINTER(dwkv_config), ctypes.POINTER(ctypes.c_size_t)],
    "dwkv_prefill_gram": [_P, _I, _P, _P, _P, _I, ctypes.c_int64, _I, _P, ctypes.c_size_t, _P],
    "dwkv_prefill_bases": [_P, _I, _I, _P, _I, _I, _P, _P, ctypes.c_size_t, _P],
    "dwkv_prefill_encode": [_P, _I, _P, _P, _P, _I, ctypes.c_int64, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "dwkv_check_errors": [_P, _P, ctypes.POINTER(ctypes.c_uint32)],
    "dwkv_clear_errors": [_P, _P],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.dwkv_strerror.argtypes = [_I]
_lib.dwkv_strerror.restype = ctypes.c_char_p
_lib.dwkv_last_hip_error.argtypes = []
_lib.dwkv_last_hip_error.restype = ctypes.c_char_p


class DwkvError(RuntimeError):
    def __init__(self, code: int, where: str):
        detail = f" [{dwkv_last_hip_error()}]" if code == DWKV_ERR_HIP else ""
        super().__init__(f"{where}: {dwkv_strerror(code)} ({code}){detail}")
        self.code = code


def dwkv_strerror(code: int) -> str:
    return _lib.dwkv_strerror(int(code)).decode()


def dwkv_last_hip_error() -> str:
    return _lib.dwkv_last_hip_error().decode()


def _check(code: int, where: str) -> None:
    if code != DWKV_OK:
        raise DwkvError(code, where)


def declared_symbols() -> Sequence[str]:
    """Entry points include/dwkv.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*\**\s*(dwkv_\w+)\s*\(", text, re.M)))


# --------------------------------------------------------------------------- helpers
def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _ptr(t, dtype=None, shape=None, name="tensor") -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return int(t.data_ptr())


def make_config(num_layers: int, layers_per_group: int, num_q_heads: int, num_kv_heads: int,
                head_dim: int, r_max: int, tier_rank: Sequence[int], tier_resid: Sequence[int],
                resid_bits: int, max_batch: int, tier_capacity: Sequence[int], max_tokens: int,
                decode_splits: int = 0, coef_bits: int = 16) -> dwkv_config:
    c = dwkv_config()
    c.num_layers, c.layers_per_group = num_layers, layers_per_group
    c.num_q_heads, c.num_kv_heads, c.head_dim, c.r_max = num_q_heads, num_kv_heads, head_dim, r_max
    c.num_tiers = len(tier_rank)
    if c.num_tiers > MAX_TIERS or len(tier_resid) != c.num_tiers or len(tier_capacity) != c.num_tiers:
        raise ValueError("tier tables must have the same length, at most 8")
    for k in range(c.num_tiers):
        c.tier_rank[k] = int(tier_rank[k])
        c.tier_resid[k] = int(tier_resid[k])
        c.tier_capacity[k] = int(tier_capacity[k])
    c.resid_bits, c.max_batch, c.decode_splits = resid_bits, max_batch, decode_splits
    c.max_tokens = int(max_tokens)
    c.coef_bits = int(coef_bits)
    return c


# --------------------------------------------------------------------------- C names
def dwkv_arena_bytes(cfg: dwkv_config) -> int:
    n = ctypes.c_size_t()
    _check(_lib.dwkv_arena_bytes(ctypes.byref(cfg), ctypes.byref(n)), "dwkv_arena_bytes")
    return n.value


def dwkv_create(cfg: dwkv_config, arena) -> ctypes.c_void_p:
    """arena: uint8 GPU tensor of at least dwkv_arena_bytes(cfg) bytes."""
    h = ctypes.c_void_p()
    size = arena.numel() * arena.element_size()
    _check(_lib.dwkv_create(ctypes.byref(cfg), _ptr(arena, name="arena"), size, ctypes.byref(h)),
           "dwkv_create")
    return h


def dwkv_destroy(h) -> None:
    _check(_lib.dwkv_destroy(h), "dwkv_destroy")


def dwkv_reset(h, stream=None) -> None:
    _check(_lib.dwkv_reset(h, _stream(stream)), "dwkv_reset")


def dwkv_set_basis(h, group: int, basisK, basisV, stream=None) -> None:
    import torch
    _check(_lib.dwkv_set_basis(h, group, _ptr(basisK, torch.float16, name="basisK"),
                               _ptr(basisV, torch.float16, name="basisV"), _stream(stream)),
           "dwkv_set_basis")


def dwkv_get_basis(h, group: int, basisK, basisV, stream=None) -> None:
    """basisK, basisV: fp16 [H_kv][r_max][d] GPU tensors, filled from the arena."""
    import torch
    _check(_lib.dwkv_get_basis(h, group, _ptr(basisK, torch.float16, name="basisK"),
                               _ptr(basisV, torch.float16, tuple(basisK.shape), name="basisV"), _stream(stream)),
           "dwkv_get_basis")


def _logical(lay: Dict[str, object]) -> dwkv_logical_layer:
    import torch
    L = dwkv_logical_layer()
    L.n_max = int(lay["tier"].shape[-1])
    L.tier = _ptr(lay["tier"], torch.uint8, name="tier")
    for z in "KV":
        ct = lay["coef" + z]
        setattr(L, "coef" + z, _ptr(ct, torch.int8 if ct.dtype == torch.int8 else torch.float16, name="coef" + z))
        if "cscale" + z in lay:
            setattr(L, "cscale" + z, _ptr(lay["cscale" + z], torch.float16, name="cscale" + z))
        setattr(L, "idx" + z, _ptr(lay["idx" + z], torch.uint8, name="idx" + z))
        setattr(L, "val" + z, _ptr(lay["val" + z], torch.int8, name="val" + z))
        setattr(L, "scale" + z, _ptr(lay["scale" + z], torch.float16, name="scale" + z))
    return L


def dwkv_import_layer(h, layer: int, lay: Dict[str, object], n_tokens: Sequence[int],
                      stream=None) -> None:
    """lay: GPU tensors in the logical form of include/dwkv.h (tier, coefK/V,
    idxK/V, valK/V, scaleK/V); n_tokens: tokens per sequence."""
    L = _logical(lay)
    n = (ctypes.c_int64 * len(n_tokens))(*[int(x) for x in n_tokens])
    _check(_lib.dwkv_import_layer(h, layer, ctypes.byref(L), n, len(n_tokens), _stream(stream)),
           "dwkv_import_layer")


def dwkv_export_layer(h, layer: int, dst: Dict[str, object], counts, slots=None, stream=None) -> None:
    import torch
    L = _logical(dst)
    batch = int(dst["tier"].shape[0])
    _check(_lib.dwkv_export_layer(h, layer, ctypes.byref(L), _ptr(counts, torch.int32, name="counts"),
                                  _ptr(slots, torch.int32, name="slots"), batch, _stream(stream)),
           "dwkv_export_layer")


def dwkv_read_counts(h, layer: int, batch: int, num_kv_heads: int, num_tiers: int,
                     stream=None) -> np.ndarray:
    out = np.zeros((batch, num_kv_heads, num_tiers), np.int32)
    _check(_lib.dwkv_read_counts(h, layer, batch, out.ctypes.data_as(ctypes.c_void_p), _stream(stream)),
           "dwkv_read_counts")
    return out


def dwkv_workspace_bytes(cfg: dwkv_config, batch: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.dwkv_workspace_bytes(ctypes.byref(cfg), batch, ctypes.byref(n)), "dwkv_workspace_bytes")
    return n.value


def dwkv_decode_splits(h) -> int:
    """Workgroups per (sequence, KV head) of this handle's decode launches."""
    n = ctypes.c_int()
    _check(_lib.dwkv_decode_splits(h, ctypes.byref(n)), "dwkv_decode_splits")
    return n.value


def dwkv_decode_attn(h, layer: int, q, out, workspace, softmax_scale: Optional[float] = None,
                     stream=None) -> None:
    """q: fp16 [B][H_q][d]; out: fp32 [B][H_q][d]; workspace: uint8 GPU tensor."""
    import torch
    B, Hq, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    ws = workspace.numel() * workspace.element_size()
    _check(_lib.dwkv_decode_attn(h, layer, _ptr(q, torch.float16, name="q"), B, float(softmax_scale),
                                 _ptr(out, torch.float32, (B, Hq, d), name="out"),
                                 _ptr(workspace, name="workspace"), ws, _stream(stream)),
           "dwkv_decode_attn")


def dwkv_append(h, layer: int, k, v, tier, gateK=None, gateV=None, stream=None) -> None:
    """k, v: fp16 [B][H_kv][d]; tier: uint8 [B][H_kv]; gates: fp16 [B][H_kv] or None."""
    import torch
    B, H, d = k.shape
    _check(_lib.dwkv_append(h, layer, _ptr(k, torch.float16, name="k"),
                            _ptr(v, torch.float16, (B, H, d), name="v"),
                            _ptr(tier, torch.uint8, (B, H), name="tier"),
                            _ptr(gateK, torch.float16, (B, H), name="gateK"),
                            _ptr(gateV, torch.float16, (B, H), name="gateV"), B, _stream(stream)),
           "dwkv_append")


def dwkv_decode_step(h, layer: int, q, out, workspace, k, v, tier, gateK=None, gateV=None,
                     softmax_scale: Optional[float] = None, stream=None) -> None:
    """dwkv_decode_attn(q) then dwkv_append(k, v, tier, gates) in one launch.
    q: fp16 [B][H_q][d]; out: fp32 [B][H_q][d]; k, v: fp16 [B][H_kv][d];
    tier: uint8 [B][H_kv]; gates: fp16 [B][H_kv] or None."""
    import torch
    B, Hq, d = q.shape
    H = k.shape[1] if k.dim() == 3 else -1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    ws = workspace.numel() * workspace.element_size()
    _check(_lib.dwkv_decode_step(h, layer, _ptr(q, torch.float16, name="q"), B, float(softmax_scale),
                                 _ptr(out, torch.float32, (B, Hq, d), name="out"),
                                 _ptr(workspace, name="workspace"), ws,
                                 _ptr(k, torch.float16, (B, H, d), name="k"),
                                 _ptr(v, torch.float16, (B, H, d), name="v"),
                                 _ptr(tier, torch.uint8, (B, H), name="tier"),
                                 _ptr(gateK, torch.float16, (B, H), name="gateK"),
                                 _ptr(gateV, torch.float16, (B, H), name="gateV"), _stream(stream)),
           "dwkv_decode_step")


def dwkv_decode_step_noalloc(h, layer: int, q, out, k, v, tier, gateK=None, gateV=None,
                             softmax_scale: Optional[float] = None, stream=None) -> None:
    """dwkv_decode_step with the library's static scratch array in place of a
    caller workspace (no device allocation anywhere).  Arguments as
    dwkv_decode_step without the workspace."""
    import torch
    B, Hq, d = q.shape
    H = k.shape[1] if k.dim() == 3 else -1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    _check(_lib.dwkv_decode_step_noalloc(h, layer, _ptr(q, torch.float16, name="q"), B, float(softmax_scale),
                                         _ptr(out, torch.float32, (B, Hq, d), name="out"),
                                         _ptr(k, torch.float16, (B, H, d), name="k"),
                                         _ptr(v, torch.float16, (B, H, d), name="v"),
                                         _ptr(tier, torch.uint8, (B, H), name="tier"),
                                         _ptr(gateK, torch.float16, (B, H), name="gateK"),
                                         _ptr(gateV, torch.float16, (B, H), name="gateV"), _stream(stream)),
           "dwkv_decode_step_noalloc")


def dwkv_materialize_layer(h, layer: int, k_out, v_out, n_out=None, stream=None) -> None:
    """k_out: fp16 [B][H_kv][n_cap][d]; v_out: fp16 [B][H_kv][n_cap/16][d][16];
    n_out: int32 [B][H_kv] or None."""
    import torch
    B, H, n_cap, d = k_out.shape
    _check(_lib.dwkv_materialize_layer(h, layer, B, _ptr(k_out, torch.float16, name="k_out"),
                                       _ptr(v_out, torch.float16, (B, H, n_cap // 16, d, 16), name="v_out"),
                                       n_cap, _ptr(n_out, torch.int32, (B, H), name="n_out"), _stream(stream)),
           "dwkv_materialize_layer")


def dwkv_dense_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                               splits: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.dwkv_dense_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, splits, ctypes.byref(n)),
           "dwkv_dense_workspace_bytes")
    return n.value


def dwkv_dense_decode(q, k, v, n_tokens, out, workspace, splits: int, softmax_scale: Optional[float] = None,
                      stream=None) -> None:
    """q fp16 [B][H_q][d]; k fp16 [B][H_kv][n_cap][d]; v fp16
    [B][H_kv][n_cap/16][d][16]; n_tokens int32 [B][H_kv]; out fp32 [B][H_q][d]."""
    import torch
    B, Hq, d = q.shape
    _, Hkv, n_cap, _ = k.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    ws = workspace.numel() * workspace.element_size()
    _check(_lib.dwkv_dense_decode(_ptr(q, torch.float16, name="q"), _ptr(k, torch.float16, name="k"),
                                  _ptr(v, torch.float16, (B, Hkv, n_cap // 16, d, 16), name="v"),
                                  _ptr(n_tokens, torch.int32, (B, Hkv), name="n_tokens"), B, Hq, Hkv, d, n_cap,
                                  splits, float(softmax_scale), _ptr(out, torch.float32, (B, Hq, d), name="out"),
                                  _ptr(workspace, name="workspace"), ws, _stream(stream)),
           "dwkv_dense_decode")


def dwkv_stream_probe(src, nbytes: int, workgroups: int, threads: int, magic: int, sink, stream=None) -> None:
    """A plain streaming read of nbytes of src (a measurement aid: the
    bandwidth one launch of that size and grid reaches)."""
    _check(_lib.dwkv_stream_probe(_ptr(src, name="src"), int(nbytes), int(workgroups), int(threads),
                                  int(magic) & 0xFFFFFFFF, _ptr(sink, torch.int32, name="sink"), _stream(stream)),
           "dwkv_stream_probe")


def dwkv_probe_workspace_bytes(cfg: dwkv_config, batch: int, n_queries: int, dense_splits: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.dwkv_probe_workspace_bytes(ctypes.byref(cfg), batch, n_queries, dense_splits, ctypes.byref(n)),
           "dwkv_probe_workspace_bytes")
    return n.value


def dwkv_probe_error(h, layer: int, q, k_ref, v_ref, n_ref, err, workspace, dense_splits: int,
                     softmax_scale: Optional[float] = None, eps: float = 1e-6, stream=None) -> None:
    """q fp16 [n_queries][B][H_q][d]; k_ref, v_ref, n_ref as dwkv_dense_decode;
    err fp32 [B][H_kv]."""
    import torch
    nq, B, Hq, d = q.shape
    _, Hkv, n_cap, _ = k_ref.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    ws = workspace.numel() * workspace.element_size()
    _check(_lib.dwkv_probe_error(h, layer, _ptr(q, torch.float16, name="q"), nq, B,
                                 _ptr(k_ref, torch.float16, name="k_ref"),
                                 _ptr(v_ref, torch.float16, (B, Hkv, n_cap // 16, d, 16), name="v_ref"),
                                 _ptr(n_ref, torch.int32, (B, Hkv), name="n_ref"), n_cap, dense_splits,
                                 float(softmax_scale), float(eps), _ptr(err, torch.float32, (B, Hkv), name="err"),
                                 _ptr(workspace, name="workspace"), ws, _stream(stream)),
           "dwkv_probe_error")


def dwkv_probe_update(tau: np.ndarray, below: np.ndarray, err: np.ndarray, tol: float, step: float,
                      patience: int, tau_min: float, tau_max: float) -> None:
    """Host arrays, updated in place: tau float32 [W], below int32 [W], err float32 [W]."""
    assert tau.dtype == np.float32 and below.dtype == np.int32 and err.dtype == np.float32
    assert tau.flags["C_CONTIGUOUS"] and below.flags["C_CONTIGUOUS"] and err.flags["C_CONTIGUOUS"]
    _check(_lib.dwkv_probe_update(tau.ctypes.data_as(ctypes.c_void_p), below.ctypes.data_as(ctypes.c_void_p),
                                  tau.size, np.ascontiguousarray(err).ctypes.data_as(ctypes.c_void_p),
                                  float(tol), float(step), int(patience), float(tau_min), float(tau_max)),
           "dwkv_probe_update")


def dwkv_prefill_workspace_bytes(cfg: dwkv_config) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.dwkv_prefill_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)), "dwkv_prefill_workspace_bytes")
    return int(out.value)


def dwkv_prefill_gram(h, layer: int, k, v, n_tokens, workspace, first: bool, stream=None) -> None:
    """k, v fp16 [B][H_kv][n_cap][d]; n_tokens int32 [B] (all on the GPU)."""
    import torch
    B, H, n_cap, d = k.shape
    _check(_lib.dwkv_prefill_gram(h, layer, _ptr(k, torch.float16, name="k"),
                                  _ptr(v, torch.float16, (B, H, n_cap, d), name="v"),
                                  _ptr(n_tokens, torch.int32, (B,), name="n_tokens"), B, n_cap, 1 if first else 0,
                                  _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                                  _stream(stream)),
           "dwkv_prefill_gram")


def dwkv_prefill_bases(h, group0: int, omega, workspace, power_iters: int = 2, ritz=None, stream=None) -> None:
    """omega fp32 [n_groups][2][H_kv][d][k]; ritz fp64 [n_groups][2][H_kv][k] or None."""
    import torch
    G, _, H, d, k = omega.shape
    _check(_lib.dwkv_prefill_bases(h, group0, G, _ptr(omega, torch.float32, name="omega"), k, power_iters,
                                   _ptr(ritz, torch.float64, (G, 2, H, k), name="ritz"),
                                   _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                                   _stream(stream)),
           "dwkv_prefill_bases")


def dwkv_prefill_encode(h, layer: int, k, v, n_tokens, tier, workspace, gateK=None, gateV=None,
                        stream=None) -> None:
    """k, v fp16 [B][H_kv][n_cap][d]; n_tokens int32 [B]; tier uint8 [B][H_kv][n_cap];
    gateK, gateV fp16 [B][H_kv][n_cap] or None."""
    import torch
    B, H, n_cap, d = k.shape
    _check(_lib.dwkv_prefill_encode(h, layer, _ptr(k, torch.float16, name="k"),
                                    _ptr(v, torch.float16, (B, H, n_cap, d), name="v"),
                                    _ptr(n_tokens, torch.int32, (B,), name="n_tokens"), B, n_cap,
                                    _ptr(tier, torch.uint8, (B, H, n_cap), name="tier"),
                                    _ptr(gateK, torch.float16, (B, H, n_cap), name="gateK"),
                                    _ptr(gateV, torch.float16, (B, H, n_cap), name="gateV"),
                                    _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                                    _stream(stream)),
           "dwkv_prefill_encode")


def dwkv_check_errors(h, stream=None) -> int:
    """Synchronises; returns the device error bits (0 when clean)."""
    bits = ctypes.c_uint32()
    rc = _lib.dwkv_check_errors(h, _stream(stream), ctypes.byref(bits))
    if rc not in (DWKV_OK, DWKV_ERR_DEVICE):
        raise DwkvError(rc, "dwkv_check_errors")
    return int(bits.value)


def dwkv_clear_errors(h, stream=None) -> None:
    _check(_lib.dwkv_clear_errors(h, _stream(stream)), "dwkv_clear_errors")
