"""Marshalling between torch tensors and the C ABI structs (pointers and shapes only)."""
from __future__ import annotations

import ctypes

import torch

from . import _abi


def ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def stream_handle(s: torch.cuda.Stream | None = None) -> int:
    s = s if s is not None else torch.cuda.current_stream()
    return s.cuda_stream


def layer_shape(shp) -> _abi.LayerShape:
    """From any object with dim, n_q_heads, n_kv_heads, head_dim, ffn_dim, max_ctx, eps, rope_theta."""
    return _abi.LayerShape(shp.dim, shp.n_q_heads, shp.n_kv_heads, shp.head_dim, shp.ffn_dim, shp.max_ctx,
                           shp.eps, shp.rope_theta)


def layer_weights(fmts: list[int], mats: list[torch.Tensor], attn_norm: torch.Tensor,
                  ffn_norm: torch.Tensor) -> _abi.LayerWeights:
    w = _abi.LayerWeights()
    for i in range(_abi.W_COUNT):
        w.fmt[i] = fmts[i]
        w.w[i] = mats[i].data_ptr()
    w.attn_norm = attn_norm.data_ptr()
    w.ffn_norm = ffn_norm.data_ptr()
    return w


def layer_layout(offsets: list[int], fmts: list[int], blob_bytes: int) -> _abi.LayerLayout:
    lay = _abi.LayerLayout()
    for i, o in enumerate(offsets):
        lay.offset[i] = o
    for i, f in enumerate(fmts):
        lay.fmt[i] = f
    lay.blob_bytes = blob_bytes
    return lay


def model_plan(shape: _abi.LayerShape, layout: _abi.LayerLayout, entries: list[tuple], skip=()):
    """entries: (blob address, tier, k_cache address, v_cache address[, fd, file offset]) per
    layer, tier a _abi.TIER_* value (True / False mean resident / pinned); skip: the layers to
    skip.  Returns (plan, keepalive); keep the second value alive while the plan is used (its
    entries' skip fields may be changed in place)."""
    arr = (_abi.LayerEntry * len(entries))()
    for i, ent in enumerate(entries):
        blob, tier, kc, vc = ent[:4]
        arr[i].blob = blob or 0
        arr[i].resident = int(tier)
        arr[i].k_cache = kc
        arr[i].v_cache = vc
        arr[i].skip = 1 if i in skip else 0
        arr[i].fd = ent[4] if len(ent) > 4 else -1
        arr[i].file_offset = ent[5] if len(ent) > 5 else 0
    plan = _abi.ModelPlan(shape, layout, len(entries), ctypes.cast(arr, ctypes.POINTER(_abi.LayerEntry)))
    return plan, arr
