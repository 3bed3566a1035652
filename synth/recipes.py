"""Shapes, format mixes and seed streams of the synthetic Llama-shaped workloads.

Shapes are the public Llama-3-8B and Llama-3.1-70B dimensions.  The pages run
Llama 8B in Q8_0 and Llama 3.1 70B in Q6_K and Q4_K_M (ntransformer overview,
de.news.hada.io, "Roadmap der Entwicklungsphasen" and "Leistung und
Caching-Struktur"; the 70B PCIe P2P article, blog.hotdry.top, §性能数据与瓶颈分析).
The Q4_K_M mix is read as Q4_K everywhere except Q6_K for attn_v and ffn_down; the
Q5_K_M mix (a format the overview lists, not a measured workload) the same with Q5_K.

Every tensor has its own seed stream, so any tensor (or any row of it) can be
regenerated alone, on either side of the comparison.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import (BLOCK_BYTES, BLOCK_ELEMS, F16, F32, Q4_K, Q5_K, Q6_K, Q8_0, fill_blocks, fill_normal_f16,
               fill_uniform_f32, matrix_bytes, normal_f32, uniform_index)

TENSORS = ("q", "k", "v", "o", "gate", "up", "down")
TID = {name: i for i, name in enumerate(TENSORS)}
TID_ATTN_NORM, TID_FFN_NORM, TID_KCACHE, TID_VCACHE = 7, 8, 9, 10
GLOBAL_LAYER = 100000  # pseudo-layer index for model-wide tensors
GID_TOKEN_EMBD, GID_OUTPUT, GID_OUTPUT_NORM, GID_H0, GID_FIRST_TOKEN, GID_X = 0, 1, 2, 3, 4, 5

GAIN_LO, GAIN_HI = 0.9, 1.1


def stream_id(layer: int, tid: int) -> int:
    return layer * 64 + tid


@dataclass(frozen=True)
class LayerShape:
    dim: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    max_ctx: int
    eps: float = 1e-5
    rope_theta: float = 500000.0

    def matrix_shape(self, name: str) -> tuple[int, int]:
        """(rows, cols) with y[rows] = W x[cols]."""
        d, q, kv, f = self.dim, self.n_q_heads * self.head_dim, self.n_kv_heads * self.head_dim, self.ffn_dim
        return {"q": (q, d), "k": (kv, d), "v": (kv, d), "o": (d, q),
                "gate": (f, d), "up": (f, d), "down": (d, f)}[name]


LLAMA3_8B = LayerShape(dim=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn_dim=14336, max_ctx=1024)
LLAMA31_70B = LayerShape(dim=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, ffn_dim=28672, max_ctx=4224)
VOCAB_70B = 128256

MIX_Q8_0 = {n: Q8_0 for n in TENSORS}
MIX_Q6_K = {n: Q6_K for n in TENSORS}
MIX_Q4_K_M = {n: (Q6_K if n in ("v", "down") else Q4_K) for n in TENSORS}
MIX_Q5_K_M = {n: (Q6_K if n in ("v", "down") else Q5_K) for n in TENSORS}
MIX_F16 = {n: F16 for n in TENSORS}  # unquantized layers (the overview lists F16 and F32 tensors)
MIX_F32 = {n: F32 for n in TENSORS}


@dataclass
class BlobLayout:
    """Byte offsets of one layer's tensors inside a contiguous layer blob."""
    offsets: dict = field(default_factory=dict)  # name -> byte offset (matrices, then the two gains)
    fmts: dict = field(default_factory=dict)
    nbytes: int = 0

    def offset_list(self) -> list[int]:
        return [self.offsets[n] for n in TENSORS] + [self.offsets["attn_norm"], self.offsets["ffn_norm"]]

    def fmt_list(self) -> list[int]:
        return [self.fmts[n] for n in TENSORS]


def _align(x: int, a: int = 256) -> int:
    return (x + a - 1) // a * a


def blob_layout(shape: LayerShape, mix: dict) -> BlobLayout:
    lay = BlobLayout()
    off = 0
    for n in TENSORS:
        r, c = shape.matrix_shape(n)
        lay.offsets[n] = off
        lay.fmts[n] = mix[n]
        off = _align(off + matrix_bytes(mix[n], r, c))
    for n in ("attn_norm", "ffn_norm"):
        lay.offsets[n] = off
        off = _align(off + 4 * shape.dim)
    lay.nbytes = off
    return lay


def layer_weight_bytes(shape: LayerShape, mix: dict) -> int:
    """Quantized weight bytes of one layer (the seven matrices only)."""
    return sum(matrix_bytes(mix[n], *shape.matrix_shape(n)) for n in TENSORS)


def fill_layer_blob(buf_addr: int, shape: LayerShape, mix: dict, layer: int, seed: int = 0,
                    layout: BlobLayout | None = None) -> BlobLayout:
    """Write layer `layer`'s seven matrices and two gains into the blob at address buf_addr."""
    lay = layout or blob_layout(shape, mix)
    for n in TENSORS:
        r, c = shape.matrix_shape(n)
        fmt = mix[n]
        fill_blocks(buf_addr + lay.offsets[n], fmt, r * (c // BLOCK_ELEMS[fmt]), seed, stream_id(layer, TID[n]))
    fill_uniform_f32(buf_addr + lay.offsets["attn_norm"], shape.dim, seed, stream_id(layer, TID_ATTN_NORM), GAIN_LO, GAIN_HI)
    fill_uniform_f32(buf_addr + lay.offsets["ffn_norm"], shape.dim, seed, stream_id(layer, TID_FFN_NORM), GAIN_LO, GAIN_HI)
    return lay


def layer_arrays(shape: LayerShape, mix: dict, layer: int, seed: int = 0) -> dict:
    """One layer as separate numpy arrays (uint8 blocks for matrices, fp32 gains)."""
    out = {}
    for n in TENSORS:
        r, c = shape.matrix_shape(n)
        buf = np.empty(matrix_bytes(mix[n], r, c), dtype=np.uint8)
        fill_blocks(buf, mix[n], buf.size // BLOCK_BYTES[mix[n]], seed, stream_id(layer, TID[n]))
        out[n] = buf
    for n, tid in (("attn_norm", TID_ATTN_NORM), ("ffn_norm", TID_FFN_NORM)):
        g = np.empty(shape.dim, dtype=np.float32)
        fill_uniform_f32(g, shape.dim, seed, stream_id(layer, tid), GAIN_LO, GAIN_HI)
        out[n] = g
    return out


def kv_cache_fill(buf_addr: int, shape: LayerShape, layer: int, which: str, n_slots: int, seed: int = 0) -> None:
    """Fill slots [0, n_slots) of every KV head of one layer's fp16 K or V cache
    ([n_kv][max_ctx][head_dim] fp16) with N(0, 1) draws; other slots untouched."""
    tid = TID_KCACHE if which == "k" else TID_VCACHE
    row = shape.max_ctx * shape.head_dim
    for g in range(shape.n_kv_heads):
        fill_normal_f16(buf_addr + 2 * g * row, n_slots * shape.head_dim, seed, stream_id(layer, tid),
                        e0=g * row)


def kv_cache_array(shape: LayerShape, layer: int, which: str, n_slots: int, seed: int = 0) -> np.ndarray:
    arr = np.zeros((shape.n_kv_heads, shape.max_ctx, shape.head_dim), dtype=np.uint16)
    kv_cache_fill(arr.ctypes.data, shape, layer, which, n_slots, seed)
    return arr


def hidden_input(dim: int, seed: int = 0) -> np.ndarray:
    return normal_f32(dim, seed, stream_id(GLOBAL_LAYER, GID_H0))


def gemv_input(cols: int, seed: int = 0) -> np.ndarray:
    return normal_f32(cols, seed, stream_id(GLOBAL_LAYER, GID_X))


def first_token(vocab: int, seed: int = 0) -> int:
    return uniform_index(vocab, seed, stream_id(GLOBAL_LAYER, GID_FIRST_TOKEN))
