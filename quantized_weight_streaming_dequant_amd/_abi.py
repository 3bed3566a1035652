"""ctypes binding of libnt.so: the same names as include/nt.h, argument marshalling only.

Every call takes device pointers as Python ints (e.g. ``tensor.data_ptr()``) and a
HIP stream handle (e.g. ``torch.cuda.current_stream().cuda_stream``); a negative
status raises NtError with the library's message.  There is no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnt.so")

Q8_0, Q4_0, Q4_K, Q6_K, Q5_K, F16, F32 = 0, 1, 2, 3, 4, 5, 6
Q4_KT = 7  # Q4_K in the library's tiles of 16 superblocks (nt_repack)
Q8_0T = 8  # Q8_0 in the library's tiles of 64 blocks (nt_repack)
Q5_KT = 9  # Q5_K in the library's tiles of 16 superblocks (nt_repack)
NT_OK, NT_EINVAL, NT_EFORMAT, NT_ESHAPE, NT_EALIGN, NT_EHOSTMEM, NT_EHIP = 0, -1, -2, -3, -4, -5, -6
W_Q, W_K, W_V, W_O, W_GATE, W_UP, W_DOWN, W_COUNT = range(8)
K_ATTN_IN, K_ATTN, K_O, K_FFN_UP, K_FFN_DOWN, K_LM_HEAD, K_GEMV, K_GEMM = range(8)
GEMM_MAX_TOK = 8
TIER_PINNED, TIER_RESIDENT, TIER_FILE = 0, 1, 2
GEMV_MAX_COLS = NT_GEMV_MAX_COLS = 32768
NT_MAX_ROWS = 1 << 30  # largest rows / vocabulary anywhere
NT_LM_HEAD_WS_BYTES = 256
NT_NOALLOC_WS_BYTES = 8 << 20  # static workspace of nt_decode_layer_noalloc
NT_MAX_CTX = 524288  # cache capacity limit (slots); KV cache max_ctx must also be a multiple of 8


class NtError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"nt error {code}: {msg}")
        self.code = code


class LayerShape(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("ffn_dim", ctypes.c_int), ("max_ctx", ctypes.c_int),
                ("eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int * W_COUNT), ("w", ctypes.c_void_p * W_COUNT),
                ("attn_norm", ctypes.c_void_p), ("ffn_norm", ctypes.c_void_p)]


class LayerLayout(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64 * (W_COUNT + 2)), ("fmt", ctypes.c_int * W_COUNT),
                ("blob_bytes", ctypes.c_int64)]


class LayerEntry(ctypes.Structure):
    _fields_ = [("blob", ctypes.c_void_p), ("resident", ctypes.c_int), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("skip", ctypes.c_int), ("fd", ctypes.c_int),
                ("file_offset", ctypes.c_int64)]


class ModelPlan(ctypes.Structure):
    _fields_ = [("shape", LayerShape), ("layout", LayerLayout), ("n_layers", ctypes.c_int),
                ("layers", ctypes.POINTER(LayerEntry))]


class StreamStats(ctypes.Structure):
    _fields_ = [("layers_streamed", ctypes.c_int64), ("h2d_bytes", ctypes.c_int64)]


class ModelHead(ctypes.Structure):
    _fields_ = [("embd_fmt", ctypes.c_int), ("token_embd", ctypes.c_void_p), ("n_vocab", ctypes.c_int64),
                ("output_norm", ctypes.c_void_p), ("out_fmt", ctypes.c_int), ("output", ctypes.c_void_p)]


_lib = None

EXPORTS = [
    "nt_last_error", "nt_version", "nt_block_elems", "nt_block_bytes", "nt_matrix_bytes", "nt_dequant", "nt_repack", "nt_gemv_q", "nt_gemm_q", "nt_layer_cosine", "nt_read_probe",
    "nt_set_stream_min_weights",
    "nt_rmsnorm", "nt_rope", "nt_attn_decode", "nt_attn_decode_ws_bytes", "nt_swiglu", "nt_decode_layer",
    "nt_decode_layer_noalloc", "nt_decode_layer_ws_bytes", "nt_decode_layer_ws_offsets", "nt_ffn_up", "nt_embed_row", "nt_argmax", "nt_stream_create",
    "nt_stream_destroy", "nt_stream_set_bounce", "nt_stream_layers", "nt_decode_token", "nt_decode_token_ws_bytes", "nt_lm_head", "nt_decode_layer_k",
    "nt_decode_layer_k_ws_bytes", "nt_decode_layer_k_ws_offsets", "nt_verify_tokens", "nt_verify_tokens_ws_bytes",
    "nt_timing_begin",
    "nt_timing_end",
]


def load(path: str = LIB_PATH):
    """Load libnt.so (once) and declare every exported signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libnt.so not found at {path}: build it with __graft_entry__.build() "
                          "or python -m quantized_weight_streaming_dequant_amd.build")
    L = ctypes.CDLL(path)
    i, i64, vp, f, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    sig = {
        "nt_last_error": ([], ctypes.c_char_p),
        "nt_version": ([], ctypes.c_char_p),
        "nt_block_elems": ([i], i),
        "nt_block_bytes": ([i], i),
        "nt_matrix_bytes": ([i, i64, i64], i64),
        "nt_dequant": ([i, i64, i64, vp, vp, vp], i),
        "nt_repack": ([i, i64, i64, vp, vp, vp], i),
        "nt_gemv_q": ([i, i64, i64, vp, vp, vp, vp], i),
        "nt_gemm_q": ([i, i64, i64, i, vp, vp, vp, vp], i),
        "nt_layer_cosine": ([i64, vp, vp, vp, vp], i),
        "nt_read_probe": ([vp, i64, vp, vp], i),
        "nt_set_stream_min_weights": ([i64], i64),
        "nt_rmsnorm": ([i64, vp, vp, f, vp, vp], i),
        "nt_rope": ([i, i, i, f, vp, vp], i),
        "nt_attn_decode": ([i, i, i, i, i, vp, vp, vp, vp, vp, sz, vp], i),
        "nt_attn_decode_ws_bytes": ([i, i, i, i], sz),
        "nt_swiglu": ([i64, vp, vp, vp, vp], i),
        "nt_decode_layer": ([ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerShape), i, vp, vp, vp, vp, sz, vp], i),
        "nt_decode_layer_ws_bytes": ([ctypes.POINTER(LayerShape)], sz),
        "nt_decode_layer_noalloc": ([ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerShape), i, vp, vp, vp, vp], i),
        "nt_ffn_up": ([ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerShape), vp, vp, vp], i),
        "nt_decode_layer_ws_offsets": ([ctypes.POINTER(LayerShape), ctypes.POINTER(ctypes.c_int64)], i),
        "nt_embed_row": ([i, i64, i64, vp, vp, vp, vp], i),
        "nt_argmax": ([i64, vp, vp, vp], i),
        "nt_stream_create": ([vp, vp, sz, ctypes.POINTER(vp)], i),
        "nt_stream_destroy": ([vp], None),
        "nt_stream_set_bounce": ([vp, vp, vp, sz, i], i),
        "nt_stream_layers": ([vp, ctypes.POINTER(ModelPlan), i, vp, vp, sz, vp, vp, ctypes.POINTER(StreamStats)], i),
        "nt_decode_token": ([vp, ctypes.POINTER(ModelPlan), ctypes.POINTER(ModelHead), i, vp, vp, vp, vp, sz, vp, vp,
                             ctypes.POINTER(StreamStats)], i),
        "nt_decode_token_ws_bytes": ([ctypes.POINTER(LayerShape)], sz),
        "nt_lm_head": ([i, i64, i64, vp, vp, f, vp, vp, vp, vp, sz, vp], i),
        "nt_decode_layer_k": ([ctypes.POINTER(LayerWeights), ctypes.POINTER(LayerShape), i, i, vp, vp, vp, vp, sz, vp],
                              i),
        "nt_decode_layer_k_ws_bytes": ([ctypes.POINTER(LayerShape), i], sz),
        "nt_decode_layer_k_ws_offsets": ([ctypes.POINTER(LayerShape), i, ctypes.POINTER(ctypes.c_int64)], i),
        "nt_verify_tokens": ([vp, ctypes.POINTER(ModelPlan), ctypes.POINTER(ModelHead), i, i, vp, vp, vp, vp, vp, sz,
                              vp, vp, ctypes.POINTER(StreamStats)], i),
        "nt_verify_tokens_ws_bytes": ([ctypes.POINTER(LayerShape), i], sz),
        "nt_timing_begin": ([i, i], i),
        "nt_timing_end": ([ctypes.POINTER(i), ctypes.POINTER(ctypes.c_double)], i),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _check(rc: int) -> int:
    if rc < 0:
        raise NtError(rc, load().nt_last_error().decode())
    return rc


def last_error() -> str:
    return load().nt_last_error().decode()


def version() -> str:
    return load().nt_version().decode()


def nt_block_elems(fmt: int) -> int:
    return _check(load().nt_block_elems(fmt))


def nt_block_bytes(fmt: int) -> int:
    return _check(load().nt_block_bytes(fmt))


def nt_matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    return _check(load().nt_matrix_bytes(fmt, rows, cols))


def nt_dequant(fmt, rows, cols, blocks, w, stream=None):
    return _check(load().nt_dequant(fmt, rows, cols, blocks, w, stream))


def nt_repack(fmt, rows, cols, src, dst, stream=None):
    return _check(load().nt_repack(fmt, rows, cols, src, dst, stream))


def nt_gemv_q(fmt, rows, cols, blocks, x, y, stream=None):
    return _check(load().nt_gemv_q(fmt, rows, cols, blocks, x, y, stream))


def nt_layer_cosine(n, a, b, out, stream=None):
    return _check(load().nt_layer_cosine(n, a, b, out, stream))


def nt_read_probe(buf, nbytes, sink, stream=None):
    return _check(load().nt_read_probe(buf, nbytes, sink, stream))


def nt_set_stream_min_weights(min_weights: int) -> int:
    """Set the GEMV launch policy's streamed-path threshold (weights per launch; < 0 leaves it);
    returns the previous value."""
    return load().nt_set_stream_min_weights(min_weights)


def nt_gemm_q(fmt, rows, cols, n_tok, blocks, x, y, stream=None):
    return _check(load().nt_gemm_q(fmt, rows, cols, n_tok, blocks, x, y, stream))


def nt_rmsnorm(n, x, gain, eps, y, stream=None):
    return _check(load().nt_rmsnorm(n, x, gain, eps, y, stream))


def nt_rope(n_heads, head_dim, pos, theta, qk, stream=None):
    return _check(load().nt_rope(n_heads, head_dim, pos, theta, qk, stream))


def nt_attn_decode_ws_bytes(n_q_heads, n_kv_heads, head_dim, max_ctx) -> int:
    return int(load().nt_attn_decode_ws_bytes(n_q_heads, n_kv_heads, head_dim, max_ctx))


def nt_attn_decode(n_q_heads, n_kv_heads, head_dim, n_ctx, max_ctx, q, k_cache, v_cache, out, ws, ws_bytes,
                   stream=None):
    return _check(load().nt_attn_decode(n_q_heads, n_kv_heads, head_dim, n_ctx, max_ctx, q, k_cache, v_cache, out,
                                        ws, ws_bytes, stream))


def nt_swiglu(n, gate, up, out, stream=None):
    return _check(load().nt_swiglu(n, gate, up, out, stream))


def nt_decode_layer(weights: LayerWeights, shape: LayerShape, pos, h, k_cache, v_cache, ws, ws_bytes, stream=None):
    return _check(load().nt_decode_layer(ctypes.byref(weights), ctypes.byref(shape), pos, h, k_cache, v_cache, ws,
                                         ws_bytes, stream))


def nt_decode_layer_noalloc(weights: LayerWeights, shape: LayerShape, pos, h, k_cache, v_cache, stream=None):
    return _check(load().nt_decode_layer_noalloc(ctypes.byref(weights), ctypes.byref(shape), pos, h, k_cache, v_cache,
                                                 stream))


def nt_ffn_up(weights: LayerWeights, shape: LayerShape, h, a, stream=None):
    return _check(load().nt_ffn_up(ctypes.byref(weights), ctypes.byref(shape), h, a, stream))


def nt_decode_layer_ws_bytes(shape: LayerShape) -> int:
    return int(load().nt_decode_layer_ws_bytes(ctypes.byref(shape)))


def nt_decode_layer_ws_offsets(shape: LayerShape) -> dict:
    off = (ctypes.c_int64 * 5)()
    _check(load().nt_decode_layer_ws_offsets(ctypes.byref(shape), off))
    return {"q": off[0], "o": off[1], "h1": off[2], "a": off[3], "part": off[4]}


def nt_embed_row(fmt, n_vocab, dim, table, token, h, stream=None):
    return _check(load().nt_embed_row(fmt, n_vocab, dim, table, token, h, stream))


def nt_argmax(n, v, out_index, stream=None):
    return _check(load().nt_argmax(n, v, out_index, stream))


def nt_stream_create(staging0, staging1, staging_bytes) -> int:
    out = ctypes.c_void_p()
    _check(load().nt_stream_create(staging0, staging1, staging_bytes, ctypes.byref(out)))
    return out.value


def nt_stream_destroy(st) -> None:
    load().nt_stream_destroy(st)


def nt_stream_set_bounce(st, bounce0, bounce1, bounce_bytes, n_threads=4):
    return _check(load().nt_stream_set_bounce(st, bounce0, bounce1, bounce_bytes, n_threads))


def nt_stream_layers(st, plan: ModelPlan, pos, h, ws, ws_bytes, compute, copy, stats: StreamStats | None = None):
    return _check(load().nt_stream_layers(st, ctypes.byref(plan), pos, h, ws, ws_bytes, compute, copy,
                                          ctypes.byref(stats) if stats is not None else None))


def nt_decode_token(st, plan: ModelPlan, head: ModelHead, pos, token, logits, h, ws, ws_bytes, compute, copy,
                    stats: StreamStats | None = None):
    return _check(load().nt_decode_token(st, ctypes.byref(plan), ctypes.byref(head), pos, token, logits, h, ws,
                                         ws_bytes, compute, copy,
                                         ctypes.byref(stats) if stats is not None else None))


def nt_decode_token_ws_bytes(shape: LayerShape) -> int:
    return int(load().nt_decode_token_ws_bytes(ctypes.byref(shape)))


def nt_decode_layer_k(weights: LayerWeights, shape: LayerShape, pos, n_tok, h, k_cache, v_cache, ws, ws_bytes,
                      stream=None):
    return _check(load().nt_decode_layer_k(ctypes.byref(weights), ctypes.byref(shape), pos, n_tok, h, k_cache, v_cache,
                                           ws, ws_bytes, stream))


def nt_decode_layer_k_ws_bytes(shape: LayerShape, n_tok: int) -> int:
    return int(load().nt_decode_layer_k_ws_bytes(ctypes.byref(shape), n_tok))


def nt_decode_layer_k_ws_offsets(shape: LayerShape, n_tok: int) -> dict:
    off = (ctypes.c_int64 * 4)()
    _check(load().nt_decode_layer_k_ws_offsets(ctypes.byref(shape), n_tok, off))
    return {"q": off[0], "o": off[1], "h1": off[2], "a": off[3]}


def nt_verify_tokens(st, plan: ModelPlan, head: ModelHead, pos, n_tok, tokens, next_tokens, logits, h, ws, ws_bytes,
                     compute, copy, stats: StreamStats | None = None):
    return _check(load().nt_verify_tokens(st, ctypes.byref(plan), ctypes.byref(head), pos, n_tok, tokens, next_tokens,
                                          logits, h, ws, ws_bytes, compute, copy,
                                          ctypes.byref(stats) if stats is not None else None))


def nt_verify_tokens_ws_bytes(shape: LayerShape, n_tok: int) -> int:
    return int(load().nt_verify_tokens_ws_bytes(ctypes.byref(shape), n_tok))


def nt_lm_head(fmt, n_vocab, dim, output, output_norm, eps, h, logits, token, ws, ws_bytes, stream=None):
    return _check(load().nt_lm_head(fmt, n_vocab, dim, output, output_norm, eps, h, logits, token, ws, ws_bytes,
                                    stream))


def nt_timing_begin(kclass: int, max_launches: int) -> None:
    _check(load().nt_timing_begin(kclass, max_launches))


def nt_timing_end() -> tuple[int, float]:
    n = ctypes.c_int()
    ms = ctypes.c_double()
    _check(load().nt_timing_end(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value
