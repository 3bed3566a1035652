"""Test-side block encoders: logical fields -> block bytes.

Written in the packing direction from the layout table (GGML block layouts,
which the ntransformer pages name but do not print), so that a decoder that
reads a field from the wrong place or with the wrong shift disagrees with it.
Only tests use this file.
"""
from __future__ import annotations

import struct

import numpy as np


def f16_bits(x: float) -> int:
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def pack_q8_0(d: float, q) -> bytes:
    q = [int(v) for v in q]
    assert len(q) == 32 and all(-128 <= v <= 127 for v in q)
    return struct.pack("<H", f16_bits(d)) + struct.pack("<32b", *q)


def pack_q4_0(d: float, n) -> bytes:
    """n: 32 unsigned nibbles; weight i is d*(n_i - 8)."""
    n = [int(v) for v in n]
    assert len(n) == 32 and all(0 <= v <= 15 for v in n)
    qs = bytes((n[i] | (n[i + 16] << 4)) for i in range(16))
    return struct.pack("<H", f16_bits(d)) + qs


def _pack_k_scales(sc, m) -> bytes:
    """The 12 bytes holding 8 six-bit (scale, min) pairs, as Q4_K and Q5_K store them."""
    s = [0] * 12
    for j in range(4):
        s[j] = sc[j] & 63          # low 6 bits: scale of sub-block j
        s[j + 4] = m[j] & 63       # low 6 bits: min of sub-block j
    for j in range(4, 8):
        s[j + 4] = (sc[j] & 15) | ((m[j] & 15) << 4)   # low nibbles of scale/min of sub-block j
        s[j - 4] |= (sc[j] >> 4) << 6                  # top two bits of the scale
        s[j] |= (m[j] >> 4) << 6                       # top two bits of the min
    return bytes(s)


def _pack_nibbles(q) -> bytes:
    """128 bytes: weight i of sub-block j = i // 32 is nibble j % 2 of byte 32 (j // 2) + i % 32."""
    qs = [0] * 128
    for i in range(256):
        j, l = i // 32, i % 32
        qs[32 * (j // 2) + l] |= (q[i] & 15) << (4 * (j % 2))
    return bytes(qs)


def pack_q4_k(d: float, dmin: float, sc, m, q) -> bytes:
    """sc, m: 8 six-bit values (one per 32-weight sub-block); q: 256 nibbles.
    Weight i = d*sc[i//32]*q[i] - dmin*m[i//32]."""
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    q = [int(v) for v in q]
    assert len(sc) == 8 and len(m) == 8 and len(q) == 256
    assert all(0 <= v < 64 for v in sc + m) and all(0 <= v < 16 for v in q)
    return struct.pack("<HH", f16_bits(d), f16_bits(dmin)) + _pack_k_scales(sc, m) + _pack_nibbles(q)


def pack_q5_k(d: float, dmin: float, sc, m, q) -> bytes:
    """sc, m: 8 six-bit values (one per 32-weight sub-block); q: 256 five-bit codes.
    Weight i = d*sc[i//32]*q[i] - dmin*m[i//32]; the fifth bit of weight i sits in bit
    i // 32 of high-bit byte i % 32."""
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    q = [int(v) for v in q]
    assert len(sc) == 8 and len(m) == 8 and len(q) == 256
    assert all(0 <= v < 64 for v in sc + m) and all(0 <= v < 32 for v in q)
    qh = [0] * 32
    for i in range(256):
        qh[i % 32] |= (q[i] >> 4) << (i // 32)
    return (struct.pack("<HH", f16_bits(d), f16_bits(dmin)) + _pack_k_scales(sc, m) + bytes(qh) +
            _pack_nibbles(q))


def pack_q6_k(d: float, s, q) -> bytes:
    """s: 16 int8 sub-scales (one per 16 weights); q: 256 six-bit codes.
    Weight i = d*s[i//16]*(q[i]-32)."""
    s = [int(v) for v in s]
    q = [int(v) for v in q]
    assert len(s) == 16 and len(q) == 256
    assert all(-128 <= v <= 127 for v in s) and all(0 <= v < 64 for v in q)
    ql = [0] * 128
    qh = [0] * 64
    for i in range(256):
        h, r = i // 128, i % 128
        k, l = r // 32, r % 32
        ql[64 * h + 32 * (k % 2) + l] |= (q[i] & 15) << (4 * (k // 2))
        qh[32 * h + l] |= (q[i] >> 4) << (2 * k)
    return bytes(ql) + bytes(qh) + struct.pack("<16b", *s) + struct.pack("<H", f16_bits(d))
