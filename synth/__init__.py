"""Seeded synthetic inputs, shared by the checker and the GPU library's callers.

This module only draws numbers: block bytes with random fields in the places
the block layouts give them, fp32 activations, fp32 norm gains and fp16 cache
entries.  It computes nothing the decode path computes.  The C generator in
``synth.c`` is built with gcc into ``libsynth.so`` next to this file.

Weights follow the distributions of the workloads on the ntransformer pages'
formats (ntransformer overview, de.news.hada.io, "Überblick über NTransformer":
GGUF formats Q4_0, Q8_0, Q4_K_M, Q5_K, Q6_K): every fp16 super-scale ~ U[0.001, 0.01],
Q8_0 codes ~ U{-127..127}, Q4_0/Q4_K/Q5_K nibbles, Q5_K high bits and Q4_K/Q5_K 6-bit
scales/mins ~ uniform, Q6_K 6-bit codes ~ uniform and int8 sub-scales ~ U{-64..63}; F16 and
F32 weights ~ N(0, 0.02), rounded to the format.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# format ids, block geometry (weights per block, bytes per block)
Q8_0, Q4_0, Q4_K, Q6_K, Q5_K, F16, F32 = 0, 1, 2, 3, 4, 5, 6
# Q4_KT, Q8_0T, Q5_KT: the library's tiled arrangements of Q4_K, Q8_0 and Q5_K bytes (made on the device from
# GGUF blocks; the generators here write GGUF blocks only)
Q4_KT, Q8_0T, Q5_KT = 7, 8, 9
FORMAT_NAMES = {Q8_0: "Q8_0", Q4_0: "Q4_0", Q4_K: "Q4_K", Q6_K: "Q6_K", Q5_K: "Q5_K", F16: "F16", F32: "F32",
                Q4_KT: "Q4_KT", Q8_0T: "Q8_0T", Q5_KT: "Q5_KT"}
# F16 and F32 tensors hold one weight per "block" (GGUF's unquantized types)
BLOCK_ELEMS = {Q8_0: 32, Q4_0: 32, Q4_K: 256, Q6_K: 256, Q5_K: 256, F16: 1, F32: 1, Q4_KT: 256, Q8_0T: 32, Q5_KT: 256}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 144, Q6_K: 210, Q5_K: 176, F16: 2, F32: 4, Q4_KT: 144, Q8_0T: 34, Q5_KT: 176}
# unquantized weights ~ N(0, F_STD): about the spread of trained Llama weight matrices (a reading:
# the pages give no distribution for them)
F_STD = 0.02

DLO, DHI = 0.001, 0.01


def build(force: bool = True) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
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
        i64, u64, vp, dbl = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
        for name in ("synth_fill_q8_0", "synth_fill_q4_0", "synth_fill_q4_k", "synth_fill_q6_k", "synth_fill_q5_k"):
            f = getattr(L, name)
            f.argtypes = [vp, i64, i64, u64, u64, dbl, dbl]
            f.restype = None
        for name in ("synth_fill_normal_f32", "synth_fill_normal_f16", "synth_fill_uniform_f32"):
            f = getattr(L, name)
            f.argtypes = [vp, i64, i64, u64, u64, dbl, dbl]
            f.restype = None
        L.synth_uniform_index.argtypes = [u64, u64, i64]
        L.synth_uniform_index.restype = i64
        L.synth_raw.argtypes = [vp, i64, i64, u64, u64]
        L.synth_raw.restype = None
        L.synth_f64_to_f16.argtypes = [dbl]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    if cols % BLOCK_ELEMS[fmt]:
        raise ValueError(f"cols={cols} is not a multiple of {BLOCK_ELEMS[fmt]} for {FORMAT_NAMES[fmt]}")
    return rows * (cols // BLOCK_ELEMS[fmt]) * BLOCK_BYTES[fmt]


def _ptr(buf) -> int:
    if isinstance(buf, np.ndarray):
        if not buf.flags["C_CONTIGUOUS"]:
            raise ValueError("buffer must be C-contiguous")
        return buf.ctypes.data
    return int(buf)  # raw address (e.g. pinned host tensor data_ptr())


def fill_blocks(buf, fmt: int, n_blocks: int, seed: int, stream: int, block0: int = 0,
                dlo: float = DLO, dhi: float = DHI) -> None:
    """Write n_blocks blocks of format fmt (blocks block0.. of the stream) at buf."""
    if fmt == F16:
        lib().synth_fill_normal_f16(_ptr(buf), block0, n_blocks, seed, stream, 0.0, F_STD)
        return
    if fmt == F32:
        lib().synth_fill_normal_f32(_ptr(buf), block0, n_blocks, seed, stream, 0.0, F_STD)
        return
    fn = {Q8_0: lib().synth_fill_q8_0, Q4_0: lib().synth_fill_q4_0,
          Q4_K: lib().synth_fill_q4_k, Q6_K: lib().synth_fill_q6_k, Q5_K: lib().synth_fill_q5_k}[fmt]
    fn(_ptr(buf), block0, n_blocks, seed, stream, dlo, dhi)


def quant_matrix(fmt: int, rows: int, cols: int, seed: int, stream: int) -> np.ndarray:
    """rows x cols matrix, row-major blocks, as a uint8 array."""
    nbytes = matrix_bytes(fmt, rows, cols)
    out = np.empty(nbytes, dtype=np.uint8)
    fill_blocks(out, fmt, nbytes // BLOCK_BYTES[fmt], seed, stream)
    return out


def quant_rows(fmt: int, cols: int, row_ids, seed: int, stream: int) -> np.ndarray:
    """Selected rows of the matrix quant_matrix(fmt, *, cols, seed, stream), regenerated alone."""
    bpr = cols // BLOCK_ELEMS[fmt]
    out = np.empty((len(row_ids), bpr * BLOCK_BYTES[fmt]), dtype=np.uint8)
    for i, r in enumerate(row_ids):
        fill_blocks(out[i], fmt, bpr, seed, stream, block0=int(r) * bpr)
    return out


def normal_f32(n: int, seed: int, stream: int, mean: float = 0.0, std: float = 1.0, e0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_fill_normal_f32(out.ctypes.data, e0, n, seed, stream, mean, std)
    return out


def normal_f16_bits(n: int, seed: int, stream: int, e0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    lib().synth_fill_normal_f16(out.ctypes.data, e0, n, seed, stream, 0.0, 1.0)
    return out


def fill_normal_f16(buf, n: int, seed: int, stream: int, e0: int = 0) -> None:
    lib().synth_fill_normal_f16(_ptr(buf), e0, n, seed, stream, 0.0, 1.0)


def uniform_f32(n: int, seed: int, stream: int, lo: float, hi: float, e0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_fill_uniform_f32(out.ctypes.data, e0, n, seed, stream, lo, hi)
    return out


def fill_uniform_f32(buf, n: int, seed: int, stream: int, lo: float, hi: float, e0: int = 0) -> None:
    lib().synth_fill_uniform_f32(_ptr(buf), e0, n, seed, stream, lo, hi)


def uniform_index(n: int, seed: int, stream: int) -> int:
    return int(lib().synth_uniform_index(seed, stream, n))


def raw(n: int, seed: int, stream: int, c0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_raw(out.ctypes.data, c0, n, seed, stream)
    return out


def f64_to_f16_bits(v: float) -> int:
    return int(lib().synth_f64_to_f16(float(v)))
