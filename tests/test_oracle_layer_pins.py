"""Closed-form pins of the checker's decode-layer composition at positions past 0 (CPU only).

The stage functions (RMSNorm, GEMV, RoPE, attention, SwiGLU) are pinned one by one in
test_oracle_pins.py.  These tests fix how oracle.decode_layer puts them together, in the
order the ntransformer overview gives the Llama layer (de.news.hada.io, "Hauptfunktionen":
RMSNorm, RoPE, GQA, KV cache, SwiGLU): RoPE turns q and k but not v, and by the angle of
the token's own position; the new key and value land in cache slot pos and are attended
to together with slots 0..pos-1; norm 1 uses attn_norm on h, norm 2 uses ffn_norm on
h1 = h + Wo o; the layer output is h1 + Wd a.

Every layer here is built from Q8_0 blocks with power-of-two scales and a handful of
nonzero integer codes, and the input is one-hot, so each stage's exact value is a closed
form: the expected outputs below are written from the construction (cos/sin/exp of known
arguments, numpy's binary16 rounding of known values), not by calling the checker's
stage functions.  tests/test_oracle_mutations.py plants mistakes in the composition and
checks that these pins catch each one.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth
from synth import recipes
from tests.blockpack import pack_q8_0

# 4 query heads over 2 KV heads (groups of 2), head_dim 32, eps 0 so that RMSNorm of a
# one-hot vector is exact
SHAPE = recipes.LayerShape(dim=64, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn_dim=64, max_ctx=16, eps=0.0,
                           rope_theta=500000.0)
MIX = {n: synth.Q8_0 for n in recipes.TENSORS}
HD = SHAPE.head_dim
H_IN = 8.0  # h = H_IN * e0


def q8_matrix(rows: int, cols: int, entries: dict, d: float = 1.0) -> np.ndarray:
    """Q8_0 blocks of a rows x cols matrix that is zero but for entries {(r, c): code};
    every block has scale d (a power of two, so every weight d * code is exact)."""
    codes = np.zeros((rows, cols), dtype=np.int64)
    for (r, c), v in entries.items():
        codes[r, c] = v
    out = bytearray()
    for r in range(rows):
        for b in range(cols // 32):
            out += pack_q8_0(d, codes[r, 32 * b:32 * b + 32])
    return np.frombuffer(bytes(out), dtype=np.uint8).copy()


def f16(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def base_weights(g1_0: float = 0.5) -> dict:
    """Zero matrices, gains 1 (attn_norm[0] = g1_0): n1 = RMSNorm(8 e0) = 8 g1_0 e0."""
    w = {}
    for n in recipes.TENSORS:
        r, c = SHAPE.matrix_shape(n)
        w[n] = q8_matrix(r, c, {})
    w["attn_norm"] = np.ones(SHAPE.dim, dtype=np.float32)
    w["attn_norm"][0] = g1_0
    w["ffn_norm"] = np.ones(SHAPE.dim, dtype=np.float32)
    return w


def caches(k_rows, v_rows):
    """K and V caches [n_kv][max_ctx][hd] as fp16 bits from per-slot float rows."""
    k = f16(k_rows).view(np.uint16).reshape(SHAPE.n_kv_heads, SHAPE.max_ctx, HD)
    v = f16(v_rows).view(np.uint16).reshape(SHAPE.n_kv_heads, SHAPE.max_ctx, HD)
    return np.ascontiguousarray(k), np.ascontiguousarray(v)


# query head h: q = A[h] (cos p, sin p) in pair 0; KV head g: k = B[g] (cos p, sin p) in pair
# 0, v = U[g]; every prefilled key is (1, 0, ..., 0), every prefilled value depends on its slot
A = (1.0, 2.0, -1.5, 0.5)
B = (1.0, -0.75)
U = ((3.0, -2.0, 1.0), (-1.0, 4.0, 0.5))


def rope_layer():
    # n1 = 4 e0 (g1_0 = 0.5); codes 4 x value with scale 1/16 in column 0 give the value itself
    w = base_weights(0.5)
    w["q"] = q8_matrix(4 * HD, 64, {(HD * h, 0): int(4 * A[h]) for h in range(4)}, d=0.0625)
    w["k"] = q8_matrix(2 * HD, 64, {(HD * g, 0): int(4 * B[g]) for g in range(2)}, d=0.0625)
    w["v"] = q8_matrix(2 * HD, 64, {(HD * g + j, 0): int(4 * U[g][j]) for g in range(2) for j in range(3)},
                       d=0.0625)
    return w


def prefill_rows():
    k = np.zeros((SHAPE.n_kv_heads, SHAPE.max_ctx, HD))
    k[:, :, 0] = 1.0
    v = np.zeros((SHAPE.n_kv_heads, SHAPE.max_ctx, HD))
    for g in range(2):
        for t in range(SHAPE.max_ctx):
            v[g, t, 0] = 0.125 * (t + 1) * (1 if g == 0 else -1)
            v[g, t, 1] = 0.25 * ((t * 5) % 7) - 0.5
            v[g, t, 2 + g] = 1.0 / (t + 2) if t % 2 else 0.0
    return k, v


def expected_rope_attention(p: int):
    """Closed forms of q, the cache entries written at slot p and the attention output."""
    cp, sp = math.cos(p), math.sin(p)  # pair 0 turns by pos * theta^0 = pos radians
    q = np.zeros(4 * HD)
    for h in range(4):
        q[HD * h], q[HD * h + 1] = A[h] * cp, A[h] * sp
    k16 = np.zeros((2, HD), dtype=np.float16)
    v16 = np.zeros((2, HD), dtype=np.float16)
    for g in range(2):
        k16[g, 0], k16[g, 1] = f16(B[g] * cp), f16(B[g] * sp)
        v16[g, :3] = f16(U[g])
    kp, vp = prefill_rows()
    o = np.zeros(4 * HD)
    for h in range(4):
        g = h // 2
        # prefilled keys (1, 0, ...): score A cos p / sqrt(hd); the new key: q . fp16(k_new)
        s = [A[h] * cp / math.sqrt(HD)] * p
        s.append((A[h] * cp * float(k16[g, 0]) + A[h] * sp * float(k16[g, 1])) / math.sqrt(HD))
        vals = [f16(vp[g, t]).astype(np.float64) for t in range(p)] + [v16[g].astype(np.float64)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        o[HD * h:HD * (h + 1)] = sum(ei / z * vi for ei, vi in zip(e, vals))
    return q, k16, v16, o


def run_layer(w, p, kc, vc, h=None):
    if h is None:
        h = np.zeros(SHAPE.dim)
        h[0] = H_IN
    return oracle.decode_layer(w, MIX, SHAPE, p, h, kc, vc)


def pin_rope_and_attention():
    w = rope_layer()
    kp, vp = prefill_rows()
    kc, vc = caches(kp, vp)
    for p in (1, 5, 11, 15):
        q, k16, v16, o = expected_rope_attention(p)
        st = run_layer(w, p, kc, vc)
        assert np.allclose(st["q"], q, rtol=0, atol=1e-13), f"q at pos {p}"
        # compared by value (a rotated zero may carry either sign)
        assert np.array_equal(np.asarray(st["k16"]).view(np.float16).reshape(2, HD), k16), f"k written at pos {p}"
        assert np.array_equal(np.asarray(st["v16"]).view(np.float16).reshape(2, HD), v16), f"v written at pos {p}"
        assert np.allclose(st["o"], o, rtol=0, atol=1e-12), f"attention output at pos {p}"


def pin_uniform_attention_is_mean_of_values():
    """Zero keys everywhere (Wk = 0, prefilled keys 0): every score is 0, so the output of each
    head is the plain mean of the values in slots 0..pos, the new value included."""
    w = rope_layer()
    w["k"] = q8_matrix(2 * HD, 64, {})
    kp, vp = prefill_rows()
    kc, vc = caches(np.zeros_like(kp), vp)
    for p in (1, 4, 9, 15):
        st = run_layer(w, p, kc, vc)
        for h in range(4):
            g = h // 2
            vals = [f16(vp[g, t]).astype(np.float64) for t in range(p)]
            new = np.zeros(HD)
            new[:3] = U[g]
            mean = (np.sum(vals, axis=0) + new) / (p + 1)
            assert np.allclose(st["o"][HD * h:HD * (h + 1)], mean, rtol=0, atol=1e-13), f"head {h} at pos {p}"


def ffn_layer():
    """Every value U0 = 2 e0 (prefill and new), so o = 2 e0 in each head; Wo o = 8 e1, so
    h1 = (8, 8, 0, ...); ffn_norm = (1, 1/2, 1, ...) gives n2 = (4 sqrt2, 2 sqrt2, 0, ...);
    gate = n2, up = (n2_0, 2 n2_1, 0, ...) -> a = (32 s(4 sqrt2), 16 s(2 sqrt2), 0, ...) with s the
    logistic; Wd moves a_0 to row 0 and a_1 to row 2."""
    w = base_weights(0.5)
    w["v"] = q8_matrix(2 * HD, 64, {(HD * g, 0): 8 for g in range(2)}, d=0.0625)  # v = 2 e0 per head
    w["o"] = q8_matrix(64, 4 * HD, {(1, 0): 4})  # row 1 reads o[0] = 2: Wo o = 8 e1
    w["ffn_norm"] = np.ones(SHAPE.dim, dtype=np.float32)
    w["ffn_norm"][1] = 0.5
    w["gate"] = q8_matrix(64, 64, {(0, 0): 1, (1, 1): 1})
    w["up"] = q8_matrix(64, 64, {(0, 0): 1, (1, 1): 2})
    w["down"] = q8_matrix(64, 64, {(0, 0): 1, (2, 1): 1})
    return w


def pin_norm2_reads_h1_and_residuals():
    w = ffn_layer()
    kp, vp = prefill_rows()
    vp[:] = 0.0
    vp[:, :, 0] = 2.0
    kc, vc = caches(kp, vp)
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    r2 = math.sqrt(2.0)
    a0 = 32.0 * sig(4 * r2)
    a1 = 16.0 * sig(2 * r2)
    for p in (3, 12):
        st = run_layer(w, p, kc, vc)
        h1 = np.zeros(SHAPE.dim)
        h1[0], h1[1] = 8.0, 8.0
        assert np.allclose(st["h1"], h1, rtol=0, atol=1e-13), f"h1 at pos {p}"
        n2 = np.zeros(SHAPE.dim)
        n2[0], n2[1] = 4 * r2, 2 * r2
        assert np.allclose(st["n2"], n2, rtol=0, atol=1e-13), f"n2 at pos {p}"
        a = np.zeros(SHAPE.ffn_dim)
        a[0], a[1] = a0, a1
        assert np.allclose(st["a"], a, rtol=0, atol=1e-12), f"a at pos {p}"
        h2 = np.zeros(SHAPE.dim)
        h2[0], h2[1], h2[2] = 8.0 + a0, 8.0, a1
        assert np.allclose(st["h2"], h2, rtol=0, atol=1e-12), f"h2 at pos {p}"


def pin_norm1_gain_and_input():
    """n1 = attn_norm * h / rms(h) on the layer's own input, with attn_norm (not ffn_norm)."""
    w = ffn_layer()
    kp, vp = prefill_rows()
    kc, vc = caches(kp, vp)
    h = np.zeros(SHAPE.dim)
    h[0], h[5] = 3.0, 4.0  # rms = 5 / 8
    st = run_layer(w, 7, kc, vc, h=h)
    n1 = np.zeros(SHAPE.dim)
    n1[0], n1[5] = 0.5 * 3.0 * 8 / 5.0, 4.0 * 8 / 5.0
    assert np.allclose(st["n1"], n1, rtol=0, atol=1e-13)


def test_rope_turns_q_and_k_at_pos_and_new_slot_is_attended():
    pin_rope_and_attention()


def test_uniform_scores_give_the_mean_of_values_including_the_new_one():
    pin_uniform_attention_is_mean_of_values()


def test_norm2_reads_h1_with_ffn_gain_and_residuals_add_up():
    pin_norm2_reads_h1_and_residuals()


def test_norm1_reads_h_with_attn_gain():
    pin_norm1_gain_and_input()


PINS = (pin_rope_and_attention, pin_uniform_attention_is_mean_of_values, pin_norm2_reads_h1_and_residuals,
        pin_norm1_gain_and_input)
