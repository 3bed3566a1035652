"""CHECKER — test infrastructure only.

A plain fp64 CPU definition of the quantized batch-1 Llama decode path, used to
judge the GPU library.  Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the GPU library never does and shares no code with it.

The arithmetic lives in ``oracle.c`` (built with gcc into ``liboracle.so``);
this file binds it and composes a decode layer and a decode token from it, in
the order the ntransformer pages give the Llama layer (ntransformer overview,
de.news.hada.io, "Hauptfunktionen": RoPE, GQA, SwiGLU, RMSNorm, KV cache).

Readings taken where the pages are silent (all listed in the design notes):
epsilon inside the square root of RMSNorm; RoPE on adjacent pairs with
theta^(-2i/d) frequencies and no frequency rescaling; KV head of query head h
is h // (n_q // n_kv); residual adds after the attention output and the FFN;
K and V enter the cache rounded to fp16 (RNE); greedy ties go to the lowest id.

Teacher forcing: every stage can be fed the GPU's captured output of the stage
before it (``forced``), so each stage is judged on its own inputs.

Pins: the C stage functions in tests/test_oracle_pins.py; the layer composition of
decode_layer at positions past 0 (RoPE on q and k only, at the token's position; the new
key and value in slot pos, attended with slots 0..pos-1; norm 2 on h1 with ffn_norm; the
residual adds) by closed forms in tests/test_oracle_layer_pins.py, which
tests/test_oracle_mutations.py shows catch 21 planted mistakes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q8_0, Q4_0, Q4_K, Q6_K, Q5_K, F16, F32 = 0, 1, 2, 3, 4, 5, 6


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, vp, dbl, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        L.or_block_elems.argtypes = [ci]
        L.or_block_elems.restype = ci
        L.or_block_bytes.argtypes = [ci]
        L.or_block_bytes.restype = ci
        L.or_f16.argtypes = [ctypes.c_uint16]
        L.or_f16.restype = dbl
        L.or_to_f16.argtypes = [dbl]
        L.or_to_f16.restype = ctypes.c_uint16
        L.or_dequant_row.argtypes = [ci, i64, vp, vp]
        L.or_dequant_row.restype = ci
        L.or_dequant_f32.argtypes = [ci, i64, i64, vp, vp]
        L.or_dequant_f32.restype = ci
        L.or_gemv.argtypes = [ci, i64, i64, vp, vp, vp, vp, vp, i64]
        L.or_gemv.restype = ci
        L.or_rmsnorm.argtypes = [i64, vp, vp, dbl, vp]
        L.or_rmsnorm.restype = None
        L.or_rope.argtypes = [ci, ci, i64, dbl, vp]
        L.or_rope.restype = None
        L.or_attn.argtypes = [ci, ci, ci, i64, i64, vp, vp, vp, vp, vp]
        L.or_attn.restype = ci
        L.or_swiglu.argtypes = [i64, vp, vp, vp, vp]
        L.or_swiglu.restype = None
        L.or_argmax.argtypes = [i64, vp]
        L.or_argmax.restype = i64
        L.or_set_threads.argtypes = [ci]
        L.or_set_threads.restype = None
        L.or_get_threads.argtypes = []
        L.or_get_threads.restype = ci
        _lib = L
    return _lib


def set_threads(n: int) -> int:
    """Set the checker's OpenMP thread count (for timing); returns the previous one."""
    old = lib().or_get_threads()
    lib().or_set_threads(int(n))
    return old


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def block_elems(fmt: int) -> int:
    return lib().or_block_elems(fmt)


def block_bytes(fmt: int) -> int:
    return lib().or_block_bytes(fmt)


def f16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib().or_f16(int(v)) for v in b], dtype=np.float64)


def to_f16_bits(v) -> np.ndarray:
    a = np.asarray(v, dtype=np.float64).ravel()
    return np.array([lib().or_to_f16(float(t)) for t in a], dtype=np.uint16)


def dequant_exact(fmt: int, rows: int, cols: int, blocks) -> np.ndarray:
    """Exact fp64 weights, rows x cols."""
    blocks = _c(blocks, np.uint8).ravel()
    out = np.empty((rows, cols), dtype=np.float64)
    rb = cols // block_elems(fmt) * block_bytes(fmt)
    for r in range(rows):
        if lib().or_dequant_row(fmt, cols, blocks[r * rb:].ctypes.data, out[r].ctypes.data) != 0:
            raise ValueError("bad format or shape")
    return out


def dequant_f32(fmt: int, rows: int, cols: int, blocks) -> np.ndarray:
    """Weights rounded once (RNE) to fp32, rows x cols."""
    blocks = _c(blocks, np.uint8).ravel()
    out = np.empty((rows, cols), dtype=np.float32)
    if lib().or_dequant_f32(fmt, rows, cols, blocks.ctypes.data, out.ctypes.data) != 0:
        raise ValueError("bad format or shape")
    return out


def gemv(fmt: int, rows: int, cols: int, blocks, x, row_idx=None):
    """(y, nrm) in fp64: y_r = sum_c w_rc x_c, nrm_r = sum_c |w_rc x_c| for the chosen rows."""
    blocks = _c(blocks, np.uint8).ravel()
    x = _c(x, np.float64).ravel()
    if x.size != cols:
        raise ValueError("x has the wrong length")
    if row_idx is None:
        n = rows
        idx_ptr = None
    else:
        idx = _c(row_idx, np.int64).ravel()
        n = idx.size
        idx_ptr = idx.ctypes.data
    y = np.empty(n, dtype=np.float64)
    nrm = np.empty(n, dtype=np.float64)
    if lib().or_gemv(fmt, rows, cols, blocks.ctypes.data, x.ctypes.data, y.ctypes.data, nrm.ctypes.data,
                     idx_ptr, n) != 0:
        raise ValueError("bad format or shape")
    return y, nrm


def gemm(fmt: int, rows: int, cols: int, blocks, X, row_idx=None):
    """(Y, NRM) in fp64 for n_tok tokens at once: row t of X (n_tok x cols) is token t's
    activation vector, and Y[t], NRM[t] are gemv() of it.  The verification pass of
    self-speculative decoding (ntransformer overview, "Hauptfunktionen") applies every
    weight matrix to all draft tokens; per token this is the plain GEMV."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    if X.shape[1] != cols:
        raise ValueError("X has the wrong width")
    out = [gemv(fmt, rows, cols, blocks, X[t], row_idx) for t in range(X.shape[0])]
    return np.stack([o[0] for o in out]), np.stack([o[1] for o in out])


def rmsnorm(x, g, eps: float) -> np.ndarray:
    x = _c(x, np.float64).ravel()
    g = _c(g, np.float64).ravel()
    y = np.empty_like(x)
    lib().or_rmsnorm(x.size, x.ctypes.data, g.ctypes.data, eps, y.ctypes.data)
    return y


def rope(x, n_heads: int, head_dim: int, pos: int, theta: float) -> np.ndarray:
    y = _c(x, np.float64).ravel().copy()
    lib().or_rope(n_heads, head_dim, pos, theta, y.ctypes.data)
    return y


def attn(q, k_cache, v_cache, n_q: int, n_kv: int, hd: int, n_ctx: int, max_ctx: int):
    """(out, nrm) fp64 over cache slots [0, n_ctx)."""
    q = _c(q, np.float64).ravel()
    kc = _c(k_cache, np.uint16).ravel()
    vc = _c(v_cache, np.uint16).ravel()
    out = np.empty(n_q * hd, dtype=np.float64)
    nrm = np.empty(n_q * hd, dtype=np.float64)
    if lib().or_attn(n_q, n_kv, hd, n_ctx, max_ctx, q.ctypes.data, kc.ctypes.data, vc.ctypes.data,
                     out.ctypes.data, nrm.ctypes.data) != 0:
        raise ValueError("bad attention shape")
    return out, nrm


def swiglu(gate, up):
    g = _c(gate, np.float64).ravel()
    u = _c(up, np.float64).ravel()
    out = np.empty_like(g)
    nrm = np.empty_like(g)
    lib().or_swiglu(g.size, g.ctypes.data, u.ctypes.data, out.ctypes.data, nrm.ctypes.data)
    return out, nrm


def cosine(a, b) -> float:
    """sum a b / sqrt(sum a^2 sum b^2) in fp64, 0 if a or b is all zeros: the similarity of a
    layer's input and output by which cosine-based layer skip ranks layers (ntransformer
    overview, "Leistung und Caching-Struktur")."""
    a = _c(a, np.float64).ravel()
    b = _c(b, np.float64).ravel()
    den = np.sqrt(np.dot(a, a) * np.dot(b, b))
    return float(np.dot(a, b) / den) if den > 0 else 0.0


def argmax(v) -> int:
    v = _c(v, np.float64).ravel()
    return int(lib().or_argmax(v.size, v.ctypes.data))


def f16_ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Distance in representable binary16 steps between finite values (sign-magnitude order)."""
    def key(b):
        b = np.asarray(b, dtype=np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)
    return np.abs(key(a_bits) - key(b_bits))


def decode_layer(w: dict, fmts: dict, shape, pos: int, h, k_cache, v_cache, forced: dict | None = None) -> dict:
    """One Llama decode layer, fp64, as a dict of every stage's output and normaliser.

    w: name -> uint8 blocks for q, k, v, o, gate, up, down; fp32 gains under
    attn_norm and ffn_norm.  k_cache / v_cache: uint16 [n_kv][max_ctx][hd]
    (copied, not modified).  forced (nullable) may hold the GPU's captured
    values: 'k16'/'v16' (fp16 bits written at slot pos; their distance in
    binary16 steps from the oracle's own rounding is reported), 'q' (post-RoPE query),
    'o' (attention output), 'h1' (hidden state after the attention residual),
    'a' (SwiGLU output).  A forced stage replaces the oracle's own value as the
    next stage's input; the oracle's own value is still reported.
    """
    forced = forced or {}
    D, nq, nkv, hd, F = shape.dim, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim
    h = np.asarray(h, dtype=np.float64)
    st = {}
    n1 = rmsnorm(h, w["attn_norm"], shape.eps)
    st["n1"] = n1
    q, nq_ = gemv(fmts["q"], nq * hd, D, w["q"], n1)
    k, nk_ = gemv(fmts["k"], nkv * hd, D, w["k"], n1)
    v, nv_ = gemv(fmts["v"], nkv * hd, D, w["v"], n1)
    q = rope(q, nq, hd, pos, shape.rope_theta)
    k = rope(k, nkv, hd, pos, shape.rope_theta)
    st.update(q=q, q_nrm=nq_, k=k, k_nrm=nk_, v=v, v_nrm=nv_)
    k16 = to_f16_bits(k)
    v16 = to_f16_bits(v)
    st.update(k16=k16, v16=v16)
    if "k16" in forced:
        fk = np.asarray(forced["k16"], dtype=np.uint16).ravel()
        fv = np.asarray(forced["v16"], dtype=np.uint16).ravel()
        st["k16_ulp"] = int(f16_ulp_distance(fk, k16).max())
        st["v16_ulp"] = int(f16_ulp_distance(fv, v16).max())
        k16, v16 = fk, fv
    kc = np.array(k_cache, dtype=np.uint16, copy=True).reshape(nkv, shape.max_ctx, hd)
    vc = np.array(v_cache, dtype=np.uint16, copy=True).reshape(nkv, shape.max_ctx, hd)
    kc[:, pos, :] = k16.reshape(nkv, hd)
    vc[:, pos, :] = v16.reshape(nkv, hd)
    q_in = np.asarray(forced["q"], dtype=np.float64) if "q" in forced else q
    o, o_nrm = attn(q_in, kc, vc, nq, nkv, hd, pos + 1, shape.max_ctx)
    st.update(o=o, o_nrm=o_nrm)
    o_in = np.asarray(forced["o"], dtype=np.float64) if "o" in forced else o
    yo, N_o = gemv(fmts["o"], D, nq * hd, w["o"], o_in)
    h1 = h + yo
    st.update(h1=h1, h1_nrm=np.abs(h) + N_o)
    h1_in = np.asarray(forced["h1"], dtype=np.float64) if "h1" in forced else h1
    n2 = rmsnorm(h1_in, w["ffn_norm"], shape.eps)
    g, N_g = gemv(fmts["gate"], F, D, w["gate"], n2)
    u, N_u = gemv(fmts["up"], F, D, w["up"], n2)
    a, N_a = swiglu(g, u)
    st.update(n2=n2, gate=g, gate_nrm=N_g, up=u, up_nrm=N_u, a=a, a_nrm=N_a)
    a_in = np.asarray(forced["a"], dtype=np.float64) if "a" in forced else a
    yd, N_d = gemv(fmts["down"], D, F, w["down"], a_in)
    h2 = h1_in + yd
    st.update(h2=h2, h2_nrm=np.abs(h1_in) + N_d, N_o=N_o, N_d=N_d)
    return st
