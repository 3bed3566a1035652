"""Pins of the fp64 checker to facts outside itself (CPU only).

Each test fixes one part of the checker against a closed form, an exact
rational brute force, an invariant, a library routine on a special case, or a
figure the pages print, chosen so that a dropped term, a wrong sign, a wrong
field offset or shift, or a transposed operand fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import recipes
from tests.blockpack import f16_bits, pack_q4_0, pack_q4_k, pack_q5_k, pack_q6_k, pack_q8_0

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- binary16

def test_f16_decode_all_codes_match_numpy():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = oracle.f16_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_f16_decode_textbook_values():
    table = {0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0001: 2.0 ** -24, 0x0400: 2.0 ** -14,
             0x3555: 0.333251953125, 0x3800: 0.5, 0x7C00: math.inf}
    for code, v in table.items():
        assert oracle.f16_to_f64([code])[0] == v


def _rounding_cases():
    vals = list(RNG.normal(0, 1, 2000)) + list(RNG.normal(0, 300, 500)) + list(RNG.uniform(-1e-4, 1e-4, 500))
    # exact ties between neighbouring binary16 values, both parities, normal and subnormal
    for code in (0x3C00, 0x3C01, 0x0001, 0x0002, 0x03FF, 0x0400, 0x7BFE):
        lo = float(np.array([code], np.uint16).view(np.float16)[0])
        hi = float(np.array([code + 1], np.uint16).view(np.float16)[0])
        vals += [(lo + hi) / 2, -(lo + hi) / 2, np.nextafter((lo + hi) / 2, 0), np.nextafter((lo + hi) / 2, 1e9)]
    vals += [65504.0, 65519.999, 65520.0, 1e6, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 0.0, -0.0]
    return np.array(vals, dtype=np.float64)


def test_f16_rounding_matches_numpy():
    vals = _rounding_cases()
    ref = vals.astype(np.float16).view(np.uint16)
    got = oracle.to_f16_bits(vals)
    assert np.array_equal(got, ref)


def test_generator_f16_rounding_matches_numpy():
    vals = _rounding_cases()
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([synth.f64_to_f16_bits(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- dequant

def test_q8_0_hand_block():
    q = [i - 16 for i in range(32)]
    blk = pack_q8_0(0.5, q)
    w = oracle.dequant_exact(synth.Q8_0, 1, 32, np.frombuffer(blk, np.uint8))[0]
    assert np.array_equal(w, 0.5 * (np.arange(32) - 16))


def test_q8_0_extremes():
    blk = pack_q8_0(-3.0, [-128, 127] * 16)
    w = oracle.dequant_exact(synth.Q8_0, 1, 32, np.frombuffer(blk, np.uint8))[0]
    assert np.array_equal(w, np.array([384.0, -381.0] * 16))


def test_q4_0_hand_block():
    n = list(range(16)) + [15 - i for i in range(16)]
    blk = pack_q4_0(2.0, n)
    w = oracle.dequant_exact(synth.Q4_0, 1, 32, np.frombuffer(blk, np.uint8))[0]
    exp = np.array([2.0 * (i - 8) for i in range(16)] + [2.0 * (7 - i) for i in range(16)])
    assert np.array_equal(w, exp)


def test_q4_k_hand_block():
    # d = 1, dmin = 0.5, scale of sub-block j = j+1, min = 2j, code_i = (i + j) mod 16
    # (j = i // 32, so neighbouring sub-blocks never share a code at the same offset)
    # -> w_i = (j+1)((i + j) mod 16) - j
    sc = [j + 1 for j in range(8)]
    m = [2 * j for j in range(8)]
    q = [(i + i // 32) % 16 for i in range(256)]
    blk = pack_q4_k(1.0, 0.5, sc, m, q)
    w = oracle.dequant_exact(synth.Q4_K, 1, 256, np.frombuffer(blk, np.uint8))[0]
    exp = np.array([(i // 32 + 1) * ((i + i // 32) % 16) - i // 32 for i in range(256)], dtype=np.float64)
    assert np.array_equal(w, exp)


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q5_K])
def test_k_scale_min_packing_exhaustive(fmt):
    """Every (scale, min) pair in 0..63 x 0..63 at every sub-block decodes back."""
    pack = pack_q4_k if fmt == synth.Q4_K else pack_q5_k
    q = [(7 * i + 3 + i // 32) % (16 if fmt == synth.Q4_K else 32) for i in range(256)]
    base_sc = [5, 9, 17, 33, 40, 51, 62, 1]
    base_m = [60, 2, 30, 44, 8, 19, 63, 27]
    d, dmin = 0.25, 0.125
    for j in range(8):
        blocks = []
        pairs = [(s, mm) for s in range(64) for mm in range(64)]
        for s, mm in pairs:
            sc = list(base_sc)
            m = list(base_m)
            sc[j], m[j] = s, mm
            blocks.append(pack(d, dmin, sc, m, q))
        buf = np.frombuffer(b"".join(blocks), np.uint8)
        w = oracle.dequant_exact(fmt, len(pairs), 256, buf)
        qa = np.array(q, dtype=np.float64)
        for r, (s, mm) in enumerate(pairs):
            sc = list(base_sc)
            m = list(base_m)
            sc[j], m[j] = s, mm
            exp = np.array([d * sc[i // 32] * qa[i] - dmin * m[i // 32] for i in range(256)])
            assert np.array_equal(w[r], exp), (j, s, mm)


def test_q5_k_hand_block():
    # d = 1, dmin = 0.5, scale of sub-block j = j+1, min = 2j, code_i = (i + 5j) mod 32
    # -> w_i = (j+1)((i + 5j) mod 32) - j; codes 16..31 set the fifth bit
    sc = [j + 1 for j in range(8)]
    m = [2 * j for j in range(8)]
    code = lambda i: (i + 5 * (i // 32)) % 32
    blk = pack_q5_k(1.0, 0.5, sc, m, [code(i) for i in range(256)])
    assert len(blk) == 176
    w = oracle.dequant_exact(synth.Q5_K, 1, 256, np.frombuffer(blk, np.uint8))[0]
    exp = np.array([(i // 32 + 1) * code(i) - i // 32 for i in range(256)], dtype=np.float64)
    assert np.array_equal(w, exp)


def test_q5_k_every_code_at_every_position():
    sc = [3, 7, 11, 13, 17, 19, 23, 29]
    code = lambda i, c: (i + c + 7 * (i // 32)) % 32
    blocks = [pack_q5_k(1.0, 0.0, sc, [0] * 8, [code(i, c) for i in range(256)]) for c in range(32)]
    w = oracle.dequant_exact(synth.Q5_K, 32, 256, np.frombuffer(b"".join(blocks), np.uint8))
    for c in range(32):
        exp = np.array([sc[i // 32] * code(i, c) for i in range(256)], dtype=np.float64)
        assert np.array_equal(w[c], exp)


def test_q5_k_is_q4_k_plus_sixteen_per_high_bit():
    """With its high bits clear a Q5_K block decodes like the Q4_K block with the same fields;
    each set high bit adds exactly 16 d sc_j to its weight and nothing elsewhere."""
    rng = np.random.default_rng(55)
    for _ in range(20):
        d, dmin = (float(np.float16(v)) for v in rng.uniform(0.001, 0.01, 2))
        sc, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        lo = rng.integers(0, 16, 256)
        hi = rng.integers(0, 2, 256)
        w4 = oracle.dequant_exact(synth.Q4_K, 1, 256, np.frombuffer(pack_q4_k(d, dmin, sc, m, lo), np.uint8))[0]
        w5_0 = oracle.dequant_exact(synth.Q5_K, 1, 256, np.frombuffer(pack_q5_k(d, dmin, sc, m, lo), np.uint8))[0]
        w5 = oracle.dequant_exact(synth.Q5_K, 1, 256, np.frombuffer(pack_q5_k(d, dmin, sc, m, lo + 16 * hi), np.uint8))[0]
        assert np.array_equal(w5_0, w4)
        assert np.array_equal(w5 - w4, 16.0 * d * np.repeat(sc, 32) * hi)


def test_q6_k_hand_block():
    # d = 0.25, sub-scale k = k - 8, code_i = (i + 11 (i // 32)) mod 64
    # -> w_i = 0.25 (i//16 - 8)(code_i - 32); every 32-run gets its own code offset
    s = [k - 8 for k in range(16)]
    code = lambda i: (i + 11 * (i // 32)) % 64
    q = [code(i) for i in range(256)]
    blk = pack_q6_k(0.25, s, q)
    w = oracle.dequant_exact(synth.Q6_K, 1, 256, np.frombuffer(blk, np.uint8))[0]
    exp = np.array([0.25 * (i // 16 - 8) * (code(i) - 32) for i in range(256)])
    assert np.array_equal(w, exp)


def test_q6_k_every_code_at_every_position():
    s = [((7 * k) % 128) - 64 for k in range(16)]
    code = lambda i, c: (i + c + 17 * (i // 32)) % 64
    blocks = [pack_q6_k(1.0, s, [code(i, c) for i in range(256)]) for c in range(64)]
    w = oracle.dequant_exact(synth.Q6_K, 64, 256, np.frombuffer(b"".join(blocks), np.uint8))
    for c in range(64):
        exp = np.array([s[i // 16] * (code(i, c) - 32) for i in range(256)], dtype=np.float64)
        assert np.array_equal(w[c], exp)


def test_q4_0_and_q8_0_every_code():
    blocks = [pack_q4_0(1.0, [(i + c) % 16 for i in range(32)]) for c in range(16)]
    w = oracle.dequant_exact(synth.Q4_0, 16, 32, np.frombuffer(b"".join(blocks), np.uint8))
    for c in range(16):
        assert np.array_equal(w[c], np.array([((i + c) % 16) - 8 for i in range(32)], dtype=np.float64))
    blocks = [pack_q8_0(1.0, [((i + 32 * c) % 256) - 128 for i in range(32)]) for c in range(8)]
    w = oracle.dequant_exact(synth.Q8_0, 8, 32, np.frombuffer(b"".join(blocks), np.uint8))
    for c in range(8):
        assert np.array_equal(w[c], np.array([((i + 32 * c) % 256) - 128 for i in range(32)], dtype=np.float64))


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q5_K])
def test_dequant_f32_is_one_rounding_of_exact(fmt):
    """fp32 output = RNE(exact rational value), checked with Fractions."""
    rows, cols = 3, 512
    blocks = synth.quant_matrix(fmt, rows, cols, seed=7, stream=fmt)
    w32 = oracle.dequant_f32(fmt, rows, cols, blocks)
    w64 = oracle.dequant_exact(fmt, rows, cols, blocks)
    # fp64 values hold at most 32 significant bits: the exact rational equals the fp64 value
    for v in w64.ravel()[::37]:
        fr = Fraction(v)
        assert fr.denominator & (fr.denominator - 1) == 0  # dyadic
        assert abs(fr.numerator).bit_length() <= 53
    assert np.array_equal(w32, w64.astype(np.float32))


def test_row_major_block_order():
    """Row r of a matrix is the r-th run of cols/block blocks; blocks run along cols."""
    rows, cols = 3, 512
    blocks = []
    for r in range(rows):
        for b in range(cols // 256):
            blocks.append(pack_q4_k(float(r + 1), 0.0, [1] * 8, [0] * 8, [b + 1] * 256))
    w = oracle.dequant_exact(synth.Q4_K, rows, cols, np.frombuffer(b"".join(blocks), np.uint8))
    for r in range(rows):
        assert np.array_equal(w[r], np.repeat([(r + 1) * 1.0, (r + 1) * 2.0], 256))


# ---------------------------------------------------------------- page figures

def test_format_sizes_match_page_figures():
    figs = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    L70 = recipes.LLAMA31_70B
    q6 = recipes.layer_weight_bytes(L70, recipes.MIX_Q6_K)
    q4m = recipes.layer_weight_bytes(L70, recipes.MIX_Q4_K_M)
    assert q6 == 701_890_560
    assert abs(q6 / 2 ** 20 - figs["q6_k_70b_layer"]["value"]) / figs["q6_k_70b_layer"]["value"] < 0.01
    # whole 70B model at Q4 (layers + embedding + output) is "about 40 GB" (read as GiB: within 5%)
    embd = synth.matrix_bytes(synth.Q4_K, recipes.VOCAB_70B, L70.dim)
    total = 80 * q4m + 2 * embd
    assert abs(total / 2 ** 30 - figs["q4_70b_weights"]["value"]) / figs["q4_70b_weights"]["value"] < 0.05
    # 26 Q6_K layers and 36 Q4_K_M layers both fit in 24 GB, and their ratio tracks the size ratio
    r = figs["resident_layers_24gb"]
    assert r["q6_k"] * q6 < r["vram_gb"] * 1e9 and r["q4_k_m"] * q4m < r["vram_gb"] * 1e9
    assert abs((r["q4_k_m"] / r["q6_k"]) / (q6 / q4m) - 1) < 0.1
    # one layer over the effective PCIe rate takes about the printed time
    p = figs["pcie_layer_time"]
    assert abs(q6 / 2 ** 20 * 1e6 / (p["effective_gbps"] * 1e9) * 1e3 - p["layer_ms"]) / p["layer_ms"] < 0.02


def test_bits_per_weight():
    bpw = {f: 8 * synth.BLOCK_BYTES[f] / synth.BLOCK_ELEMS[f] for f in synth.BLOCK_BYTES}
    assert bpw == {synth.Q8_0: 8.5, synth.Q4_0: 4.5, synth.Q4_K: 4.5, synth.Q6_K: 6.5625, synth.Q5_K: 5.5,
                   synth.F16: 16.0, synth.F32: 32.0, synth.Q4_KT: 4.5, synth.Q8_0T: 8.5, synth.Q5_KT: 5.5}
    # the checker knows the pages' formats; Q4_KT is the library's arrangement of Q4_K bytes
    for f in (synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q5_K, synth.F16, synth.F32):
        assert oracle.block_bytes(f) == synth.BLOCK_BYTES[f]
        assert oracle.block_elems(f) == synth.BLOCK_ELEMS[f]


# ---------------------------------------------------------------- F16 / F32 weights

def test_f16_weights_every_code_is_its_binary16_value():
    """An F16 tensor is its weights as IEEE binary16: every one of the 65536 codes decodes to
    numpy's value (NaNs as NaN, both zeros), and the fp32 dequantization is that value exactly."""
    codes = np.arange(65536, dtype=np.uint16)
    w = oracle.dequant_exact(synth.F16, 1, 65536, codes.view(np.uint8))[0]
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(w), nan) and np.array_equal(w[~nan], ref[~nan])
    assert math.copysign(1.0, w[0x8000]) == -1.0 and w[0x7C00] == math.inf and w[0xFC00] == -math.inf
    w32 = oracle.dequant_f32(synth.F16, 256, 256, codes.view(np.uint8))
    ref32 = codes.view(np.float16).astype(np.float32).reshape(256, 256)
    assert np.array_equal(np.isnan(w32), np.isnan(ref32))
    assert np.array_equal(w32[~np.isnan(ref32)], ref32[~np.isnan(ref32)])


def test_f32_weights_hand_values():
    vals = np.array([1.0, -2.5, 3.4028234663852886e38, 1.401298464324817e-45, -0.0, 0.1, 65504.0, -1e-30,
                     np.float32(np.pi)], dtype=np.float32)
    w = oracle.dequant_exact(synth.F32, 1, vals.size, vals.view(np.uint8))[0]
    assert np.array_equal(w, vals.astype(np.float64)) and math.copysign(1.0, w[4]) == -1.0
    assert w[2] == 2.0 ** 128 - 2.0 ** 104 and w[3] == 2.0 ** -149  # largest normal, smallest subnormal
    rnd = synth.quant_matrix(synth.F32, 3, 1000, seed=1, stream=3)
    assert np.array_equal(oracle.dequant_f32(synth.F32, 3, 1000, rnd), rnd.view(np.float32).reshape(3, 1000))


def test_f16_f32_geometry_and_generator():
    assert (oracle.block_elems(synth.F16), oracle.block_bytes(synth.F16)) == (1, 2)
    assert (oracle.block_elems(synth.F32), oracle.block_bytes(synth.F32)) == (1, 4)
    w = synth.quant_matrix(synth.F16, 64, 4096, seed=0, stream=5).view(np.float16).astype(np.float64)
    assert abs(w.std() - synth.F_STD) < 0.02 * synth.F_STD and abs(w.mean()) < 0.02 * synth.F_STD
    # rows regenerate alone
    rows = synth.quant_rows(synth.F32, 512, [3, 17], 0, 9)
    full = synth.quant_matrix(synth.F32, 20, 512, 0, 9).reshape(20, -1)
    assert np.array_equal(rows[0], full[3]) and np.array_equal(rows[1], full[17])


# ---------------------------------------------------------------- GEMV

@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q5_K, synth.F16, synth.F32])
def test_gemv_exact_rational_brute_force(fmt):
    rows, cols = 4, 512
    blocks = synth.quant_matrix(fmt, rows, cols, seed=3, stream=10 + fmt)
    x = synth.normal_f32(cols, seed=3, stream=20 + fmt).astype(np.float64)
    y, nrm = oracle.gemv(fmt, rows, cols, blocks, x)
    w = oracle.dequant_exact(fmt, rows, cols, blocks)
    for r in range(rows):
        exact = sum(Fraction(w[r, c]) * Fraction(x[c]) for c in range(cols))
        n_exact = sum(abs(Fraction(w[r, c]) * Fraction(x[c])) for c in range(cols))
        assert abs(Fraction(y[r]) - exact) <= Fraction(cols) * Fraction(2) ** -52 * n_exact
        assert abs(Fraction(nrm[r]) - n_exact) <= Fraction(cols) * Fraction(2) ** -52 * n_exact


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q5_K, synth.F16, synth.F32])
def test_gemv_one_hot_picks_a_column(fmt):
    rows, cols = 5, 512
    blocks = synth.quant_matrix(fmt, rows, cols, seed=4, stream=30 + fmt)
    w = oracle.dequant_exact(fmt, rows, cols, blocks)
    for j in (0, 1, 31, 32, 255, 256, 300, 511):
        x = np.zeros(cols)
        x[j] = 1.0
        y, nrm = oracle.gemv(fmt, rows, cols, blocks, x)
        assert np.array_equal(y, w[:, j])
        assert np.array_equal(nrm, np.abs(w[:, j]))


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q8_0])
def test_gemm_token_t_is_row_t(fmt):
    """Token t of X is X's row t and lands in Y's row t: one-hot tokens pick their columns."""
    rows, cols = 6, 512
    blocks = synth.quant_matrix(fmt, rows, cols, seed=6, stream=50 + fmt)
    w = oracle.dequant_exact(fmt, rows, cols, blocks)
    picks = [5, 300, 0, 511, 37]
    X = np.zeros((len(picks), cols))
    for t, c in enumerate(picks):
        X[t, c] = 2.0 ** -t
    Y, N = oracle.gemm(fmt, rows, cols, blocks, X)
    assert Y.shape == (len(picks), rows)
    for t, c in enumerate(picks):
        assert np.array_equal(Y[t], w[:, c] * 2.0 ** -t)
        assert np.array_equal(N[t], np.abs(w[:, c]) * 2.0 ** -t)


def test_gemv_constant_blocks_and_zero_x():
    # every weight equal: y = w * sum(x)
    blk = pack_q8_0(0.25, [3] * 32)
    blocks = np.frombuffer(blk * 16, np.uint8)  # 2 rows x 256 cols
    x = RNG.normal(size=256)
    y, _ = oracle.gemv(synth.Q8_0, 2, 256, blocks, x)
    assert np.allclose(y, 0.75 * x.sum(), rtol=1e-14, atol=1e-14)
    y0, n0 = oracle.gemv(synth.Q8_0, 2, 256, blocks, np.zeros(256))
    assert np.all(y0 == 0) and np.all(n0 == 0)


def test_gemv_row_subset_matches_full():
    fmt, rows, cols = synth.Q6_K, 9, 512
    blocks = synth.quant_matrix(fmt, rows, cols, seed=5, stream=40)
    x = RNG.normal(size=cols)
    y, nrm = oracle.gemv(fmt, rows, cols, blocks, x)
    ys, ns = oracle.gemv(fmt, rows, cols, blocks, x, row_idx=[8, 0, 3])
    assert np.array_equal(ys, y[[8, 0, 3]]) and np.array_equal(ns, nrm[[8, 0, 3]])


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_unit_rms_at_eps0_and_scale_invariance():
    x = RNG.normal(size=4096) * 3.7
    g = np.ones(4096)
    y = oracle.rmsnorm(x, g, 0.0)
    assert abs(np.sqrt(np.mean(y ** 2)) - 1.0) < 1e-14
    assert np.allclose(oracle.rmsnorm(x * 1234.5, g, 0.0), y, rtol=1e-13, atol=0)
    gg = RNG.uniform(0.9, 1.1, 4096)
    assert np.allclose(oracle.rmsnorm(x, gg, 0.0), gg * y, rtol=1e-14, atol=0)


def test_rmsnorm_eps_inside_root():
    x = RNG.normal(size=64) * 0.01
    eps = 1e-5
    y = oracle.rmsnorm(x, np.ones(64), eps)
    ms = np.mean(x ** 2)
    assert abs(np.sqrt(np.mean(y ** 2)) - np.sqrt(ms / (ms + eps))) < 1e-14
    # n = 1 closed form
    assert abs(oracle.rmsnorm([2.0], [1.5], 0.25)[0] - 1.5 * 2.0 / math.sqrt(4.25)) < 1e-15


# ---------------------------------------------------------------- RoPE

HD = 128


def test_rope_identity_at_pos0_and_norms():
    x = RNG.normal(size=4 * HD)
    assert np.array_equal(oracle.rope(x, 4, HD, 0, 5e5), x)
    y = oracle.rope(x, 4, HD, 4223, 5e5)
    pn = lambda v: np.hypot(v[0::2], v[1::2])
    assert np.allclose(pn(y), pn(x), rtol=1e-14, atol=0)


def test_rope_pair0_turns_by_pos_radians_and_pairs_are_adjacent():
    pos = 1023
    x = np.zeros(HD)
    x[0] = 1.0
    y = oracle.rope(x, 1, HD, pos, 5e5)
    assert abs(y[0] - math.cos(pos)) < 1e-13 and abs(y[1] - math.sin(pos)) < 1e-13
    assert np.all(y[2:] == 0)
    # pair 32 of 64 turns by pos / sqrt(theta) (its frequency is theta^(-1/2))
    x = np.zeros(HD)
    x[64] = 1.0
    y = oracle.rope(x, 1, HD, 1, 5e5)
    a = 1 / math.sqrt(5e5)
    assert abs(y[64] - math.cos(a)) < 1e-15 and abs(y[65] - math.sin(a)) < 1e-15
    assert np.count_nonzero(y) == 2


def test_rope_composes_and_is_relative():
    x = RNG.normal(size=HD)
    k = RNG.normal(size=HD)
    a = oracle.rope(oracle.rope(x, 1, HD, 700, 5e5), 1, HD, 300, 5e5)
    b = oracle.rope(x, 1, HD, 1000, 5e5)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    d1 = np.dot(oracle.rope(x, 1, HD, 4100, 5e5), oracle.rope(k, 1, HD, 4000, 5e5))
    d2 = np.dot(oracle.rope(x, 1, HD, 150, 5e5), oracle.rope(k, 1, HD, 50, 5e5))
    assert abs(d1 - d2) < 1e-10 * (np.abs(x) @ np.abs(k))


# ---------------------------------------------------------------- attention

def _f16(a):
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def test_attention_matches_torch_sdpa_with_gqa():
    n_q, n_kv, hd, max_ctx, n_ctx = 8, 2, 32, 40, 37
    q = RNG.normal(size=n_q * hd)
    kc = _f16(RNG.normal(size=(n_kv, max_ctx, hd)))
    vc = _f16(RNG.normal(size=(n_kv, max_ctx, hd)))
    out, nrm = oracle.attn(q, kc, vc, n_q, n_kv, hd, n_ctx, max_ctx)
    K = torch.from_numpy(kc.view(np.float16).astype(np.float64))[:, :n_ctx]
    V = torch.from_numpy(vc.view(np.float16).astype(np.float64))[:, :n_ctx]
    K = K.repeat_interleave(n_q // n_kv, dim=0)
    V = V.repeat_interleave(n_q // n_kv, dim=0)
    Q = torch.from_numpy(q.reshape(n_q, 1, hd))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).reshape(-1).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
    assert np.all(nrm >= np.abs(out) - 1e-12)


def test_attention_special_cases():
    n_q, n_kv, hd, max_ctx = 4, 2, 16, 8
    q = RNG.normal(size=n_q * hd)
    vc = _f16(RNG.normal(size=(n_kv, max_ctx, hd)))
    kc = _f16(RNG.normal(size=(n_kv, max_ctx, hd)))
    # one key: output is that value row
    out, _ = oracle.attn(q, kc, vc, n_q, n_kv, hd, 1, max_ctx)
    v0 = vc.view(np.float16).astype(np.float64)[:, 0]
    assert np.allclose(out.reshape(n_q, hd), np.repeat(v0, 2, axis=0), rtol=0, atol=1e-15)
    # identical keys: output is the mean of the values
    kc_same = np.repeat(kc[:, :1], max_ctx, axis=1)
    out, _ = oracle.attn(q, kc_same, vc, n_q, n_kv, hd, 6, max_ctx)
    vm = vc.view(np.float16).astype(np.float64)[:, :6].mean(axis=1)
    assert np.allclose(out.reshape(n_q, hd), np.repeat(vm, 2, axis=0), rtol=0, atol=1e-13)
    # one dominant key: its value wins
    kd = kc.view(np.float16).astype(np.float64).copy()
    qd = np.tile(np.ones(hd), n_q)
    kd[:, :, :] = 0.0
    kd[:, 3, :] = 60.0
    out, _ = oracle.attn(qd, _f16(kd), vc, n_q, n_kv, hd, 6, max_ctx)
    v3 = vc.view(np.float16).astype(np.float64)[:, 3]
    assert np.allclose(out.reshape(n_q, hd), np.repeat(v3, 2, axis=0), rtol=0, atol=1e-12)


def test_attention_group_mapping():
    """Only KV head 1 holds nonzero values: exactly query heads 2..3 (of 4, 2 KV heads) see them."""
    n_q, n_kv, hd, max_ctx = 4, 2, 8, 4
    q = RNG.normal(size=n_q * hd)
    kc = _f16(RNG.normal(size=(n_kv, max_ctx, hd)))
    v = np.zeros((n_kv, max_ctx, hd))
    v[1] = 1.0
    out, _ = oracle.attn(q, kc, _f16(v), n_q, n_kv, hd, 4, max_ctx)
    out = out.reshape(n_q, hd)
    assert np.all(out[:2] == 0) and np.allclose(out[2:], 1.0, rtol=0, atol=1e-15)


# ---------------------------------------------------------------- SwiGLU

def test_swiglu_matches_torch_silu_and_limits():
    g = np.concatenate([RNG.normal(size=1000) * 5, [0.0, 100.0, -100.0, 800.0, -800.0]])
    u = RNG.normal(size=g.size)
    out, nrm = oracle.swiglu(g, u)
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.all(np.isfinite(out))
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-300)
    assert out[1000] == 0.0
    assert np.all(nrm >= np.abs(out))


def test_cosine_closed_forms():
    a = RNG.normal(size=1000)
    assert abs(oracle.cosine(a, a) - 1.0) < 1e-15
    assert abs(oracle.cosine(a, -a) + 1.0) < 1e-15
    assert abs(oracle.cosine(3.0 * a, 0.5 * a) - 1.0) < 1e-15
    assert oracle.cosine(a, np.zeros(1000)) == 0.0 and oracle.cosine(np.zeros(3), np.zeros(3)) == 0.0
    # the angle in a plane
    for th in (0.0, 0.3, 1.0, math.pi / 2, 2.5, math.pi):
        assert abs(oracle.cosine([1.0, 0.0], [math.cos(th), math.sin(th)]) - math.cos(th)) < 1e-15
    # orthogonal by construction: b minus its projection on a
    b = RNG.normal(size=1000)
    b -= a * (b @ a) / (a @ a)
    assert abs(oracle.cosine(a, b)) < 1e-12
    # scale invariance and symmetry on unrelated vectors, against the textbook formula by hand
    c = RNG.normal(size=1000)
    ref = sum(x * y for x, y in zip(a, c)) / math.sqrt(sum(x * x for x in a) * sum(y * y for y in c))
    assert abs(oracle.cosine(a, c) - ref) < 1e-12 and abs(oracle.cosine(c, 7.0 * a) - ref) < 1e-12


def test_argmax_ties_lowest():
    assert oracle.argmax([1.0, 3.0, 3.0, -1.0]) == 1
    assert oracle.argmax([-5.0]) == 0


# ---------------------------------------------------------------- layer

SMALL = recipes.LayerShape(dim=512, n_q_heads=8, n_kv_heads=2, head_dim=64, ffn_dim=768, max_ctx=16)


def _small_layer(mix, zero=()):
    w = recipes.layer_arrays(SMALL, mix, layer=0, seed=11)
    for n in zero:
        w[n] = np.zeros_like(w[n])  # all-zero blocks: d = 0, every weight 0
    return w


def test_layer_zero_output_projections_is_identity():
    w = _small_layer(recipes.MIX_Q4_K_M, zero=("o", "down"))
    kc = recipes.kv_cache_array(SMALL, 0, "k", 16)
    vc = recipes.kv_cache_array(SMALL, 0, "v", 16)
    h = RNG.normal(size=SMALL.dim)
    st = oracle.decode_layer(w, recipes.MIX_Q4_K_M, SMALL, 9, h, kc, vc)
    assert np.array_equal(st["h2"], h)


def test_layer_forcing_own_values_changes_nothing():
    w = _small_layer(recipes.MIX_Q8_0)
    kc = recipes.kv_cache_array(SMALL, 0, "k", 16)
    vc = recipes.kv_cache_array(SMALL, 0, "v", 16)
    h = RNG.normal(size=SMALL.dim)
    st = oracle.decode_layer(w, recipes.MIX_Q8_0, SMALL, 15, h, kc, vc)
    st2 = oracle.decode_layer(w, recipes.MIX_Q8_0, SMALL, 15, h, kc, vc,
                              forced={"k16": st["k16"], "v16": st["v16"], "q": st["q"], "o": st["o"],
                                      "h1": st["h1"], "a": st["a"]})
    assert np.array_equal(st["h2"], st2["h2"]) and st2["k16_ulp"] == 0


def test_layer_residual_paths_match_stage_calls():
    """h2 = h + Wo o + Wd a with the stages called one by one."""
    mix = recipes.MIX_Q4_K_M
    w = _small_layer(mix)
    kc = recipes.kv_cache_array(SMALL, 0, "k", 16)
    vc = recipes.kv_cache_array(SMALL, 0, "v", 16)
    h = RNG.normal(size=SMALL.dim)
    st = oracle.decode_layer(w, mix, SMALL, 5, h, kc, vc)
    yo, _ = oracle.gemv(mix["o"], SMALL.dim, SMALL.n_q_heads * SMALL.head_dim, w["o"], st["o"])
    yd, _ = oracle.gemv(mix["down"], SMALL.dim, SMALL.ffn_dim, w["down"], st["a"])
    assert np.allclose(st["h2"], h + yo + yd, rtol=1e-13, atol=1e-12)
    # the new key/value pair is written at slot pos and attended to: with pos = 0 the output is v
    st0 = oracle.decode_layer(w, mix, SMALL, 0, h, kc, vc)
    v16 = st0["v16"].view(np.float16).astype(np.float64).reshape(SMALL.n_kv_heads, SMALL.head_dim)
    assert np.allclose(st0["o"].reshape(SMALL.n_q_heads, -1), np.repeat(v16, 4, axis=0), atol=1e-15, rtol=0)
