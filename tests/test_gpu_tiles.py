"""GPU parity of the tiled layouts NT_Q4_KT and NT_Q8_0T (MI355X only), through the C ABI.

nt_repack rearranges Q4_K matrices (GGUF's block order; the overview, de.news.hada.io,
"Überblick über NTransformer", names Q4_K_M) into tiles of 16 superblocks whose 16-byte
parts the GEMV's lanes read as whole cache lines.  The layout is the library's own; the
weights are not changed.  Checked here:
  * the repacked bytes against the layout as include/nt.h states it, restated in numpy;
  * nt_dequant of the tiled matrix bit-exact against the checker's Q4_K dequantization;
  * the GEMV, the greedy LM head, the embedding row and the fused decode layer in the tiled
    layout bit for bit equal to the same calls on the Q4_K matrices (the kernels run the same
    arithmetic on the same weights; only the addresses of the loads differ), and the GEMV
    and the k-token GEMM within the tolerance of the checker.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import quantized_weight_streaming_dequant_amd as nt
import synth
from quantized_weight_streaming_dequant_amd import torch_glue as tg
from synth import recipes
from tests.gpu_util import check_rel, dev, host, same_value, say, stream, v_to_device

pytestmark = pytest.mark.gpu

Q4K, Q4KT = synth.Q4_K, synth.Q4_KT


def tiles_layout(blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The NT_Q4_KT bytes of a Q4_K matrix as include/nt.h describes them: per row, tiles of
    16 superblocks (m in the last), headers first, then the first and the second 16 code bytes
    of each quarter g of each superblock j, in (j, g) order."""
    nsb = cols // 256
    b = blocks.reshape(rows, nsb, 144)
    out = np.empty((rows, nsb * 144), np.uint8)
    for t0 in range(0, nsb, 16):
        m = min(16, nsb - t0)
        tile = b[:, t0:t0 + m]
        base = 144 * t0
        out[:, base:base + 16 * m] = tile[:, :, :16].reshape(rows, -1)
        qs = tile[:, :, 16:].reshape(rows, m, 4, 2, 16)  # quarter g: bytes 32g + 16 half + i
        out[:, base + 16 * m:base + 80 * m] = qs[:, :, :, 0, :].reshape(rows, -1)
        out[:, base + 80 * m:base + 144 * m] = qs[:, :, :, 1, :].reshape(rows, -1)
    return out.ravel()


def repack(rows: int, cols: int, src: torch.Tensor) -> torch.Tensor:
    dst = torch.empty_like(src)
    nt.nt_repack(Q4KT, rows, cols, src.data_ptr(), dst.data_ptr(), stream())
    return dst


def gemv(fmt, rows, cols, w: torch.Tensor, xd: torch.Tensor) -> np.ndarray:
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    nt.nt_gemv_q(fmt, rows, cols, w.data_ptr(), xd.data_ptr(), y.data_ptr(), stream())
    return host(y)


# whole tiles, a last tile of one superblock, a row of one partial tile, the 70B shapes
SHAPES = [(1, 256), (7, 768), (3, 4096), (2, 4352), (3, 3840), (5, 28672), (33, 8192 + 256 * 7)]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_repack_layout_and_dequant_bit_exact(rows, cols):
    say(f"repack Q4_K -> Q4_KT {rows}x{cols}")
    blocks = synth.quant_matrix(Q4K, rows, cols, seed=3, stream=1200)
    t = repack(rows, cols, dev(blocks))
    assert np.array_equal(host(t), tiles_layout(blocks, rows, cols))
    w = torch.empty(rows * cols, dtype=torch.float32, device="cuda")
    nt.nt_dequant(Q4KT, rows, cols, t.data_ptr(), w.data_ptr(), stream())
    assert same_value(host(w).reshape(rows, cols), oracle.dequant_f32(Q4K, rows, cols, blocks))


GEMV_SHAPES = [(1, 256), (23, 1280), (130, 4352), (3, 12288), (64, 3840), (8192, 8192), (1024, 8192),
               (28672, 8192), (8192, 28672), (64, nt.NT_GEMV_MAX_COLS)]


@pytest.mark.parametrize("rows,cols", GEMV_SHAPES)
def test_gemv_tiled_equals_q4_k_and_matches_oracle(rows, cols):
    say(f"gemv Q4_KT {rows}x{cols}")
    blocks = synth.quant_matrix(Q4K, rows, cols, seed=0, stream=1300)
    x = synth.normal_f32(cols, seed=0, stream=1301)
    w = dev(blocks)
    xd = dev(x)
    y_k = gemv(Q4K, rows, cols, w, xd)
    y_t = gemv(Q4KT, rows, cols, repack(rows, cols, w), xd)
    assert np.array_equal(y_t.view(np.uint32), y_k.view(np.uint32))
    ref, nrm = oracle.gemv(Q4K, rows, cols, blocks, x.astype(np.float64))
    worst = check_rel(y_t, ref, nrm, what=f"Q4_KT {rows}x{cols}")
    say(f"  worst rel err {worst:.2e}")


# one token, two (the VALU GEMM at every count: the matrix cores do not take the tiled
# layout), column chunks that start at tile boundaries (the widest x, 65 superblocks)
GEMM_CASES = [(1, 256, 1), (17, 512, 4), (130, 4352, 6), (300, 16640, 5), (40, 32768, 8), (1024, 8192, 2),
              (512, 8192, 8)]


@pytest.mark.parametrize("rows,cols,n_tok", GEMM_CASES)
def test_gemm_tiled_matches_oracle(rows, cols, n_tok):
    say(f"gemm Q4_KT {rows}x{cols} x {n_tok}")
    blocks = synth.quant_matrix(Q4K, rows, cols, seed=8, stream=1400)
    X = np.stack([synth.normal_f32(cols, seed=8, stream=1401 + t) for t in range(n_tok)])
    w = repack(rows, cols, dev(blocks))
    xd = dev(X.astype(np.float32))
    Y = torch.empty(n_tok * rows, dtype=torch.float32, device="cuda")
    nt.nt_gemm_q(Q4KT, rows, cols, n_tok, w.data_ptr(), xd.data_ptr(), Y.data_ptr(), stream())
    Y = host(Y).reshape(n_tok, rows)
    ref, nrm = oracle.gemm(Q4K, rows, cols, blocks, X.astype(np.float64))
    for t in range(n_tok):
        check_rel(Y[t], ref[t], nrm[t], what=f"Q4_KT {rows}x{cols} token {t}")


def test_embed_row_tiled_equals_q4_k():
    vocab, dim = 1000, 4352
    say(f"embedding rows Q4_KT {vocab}x{dim}")
    table = dev(synth.quant_matrix(Q4K, vocab, dim, seed=4, stream=1500))
    tiled = repack(vocab, dim, table)
    for tok in (0, 1, 517, vocab - 1):
        t = torch.tensor([tok], dtype=torch.int32, device="cuda")
        a = torch.empty(dim, dtype=torch.float32, device="cuda")
        b = torch.empty(dim, dtype=torch.float32, device="cuda")
        nt.nt_embed_row(Q4K, vocab, dim, table.data_ptr(), t.data_ptr(), a.data_ptr(), stream())
        nt.nt_embed_row(Q4KT, vocab, dim, tiled.data_ptr(), t.data_ptr(), b.data_ptr(), stream())
        assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32)), tok


@pytest.mark.parametrize("vocab,dim", [(1000, 1024), (128256, 8192)])
def test_lm_head_tiled_equals_q4_k(vocab, dim):
    say(f"LM head Q4_KT {vocab}x{dim}")
    out = dev(synth.quant_matrix(Q4K, vocab, dim, seed=5, stream=1600))
    tiled = repack(vocab, dim, out)
    onorm = dev(synth.uniform_f32(dim, 5, 1601, 0.9, 1.1))
    h = dev(synth.normal_f32(dim, seed=5, stream=1602))
    res = []
    for fmt, w in ((Q4K, out), (Q4KT, tiled)):
        logits = torch.empty(vocab, dtype=torch.float32, device="cuda")
        tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        ws = torch.zeros(nt.NT_LM_HEAD_WS_BYTES, dtype=torch.uint8, device="cuda")
        nt.nt_lm_head(fmt, vocab, dim, w.data_ptr(), onorm.data_ptr(), 1e-5, h.data_ptr(), logits.data_ptr(),
                      tok.data_ptr(), ws.data_ptr(), ws.numel(), stream())
        torch.cuda.synchronize()
        res.append((int(tok.item()), host(logits).copy()))
    assert res[0][0] == res[1][0]
    assert np.array_equal(res[0][1].view(np.uint32), res[1][1].view(np.uint32))


SMALL = recipes.LayerShape(dim=1024, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn_dim=2816, max_ctx=96)


@pytest.mark.parametrize("shape,pos", [(SMALL, 0), (SMALL, 77), (recipes.LLAMA31_70B, 4096)])
def test_decode_layer_tiled_equals_q4_k(shape, pos):
    """The fused layer with its Q4_K matrices (q, k, o, gate, up of the Q4_K_M mix) tiled gives
    h, the new K and V and every stage in the workspace bit for bit as with the Q4_K ones."""
    say(f"decode layer Q4_K_M with tiled Q4_K, dim={shape.dim} pos={pos}")
    mix = recipes.MIX_Q4_K_M
    arrays = recipes.layer_arrays(shape, mix, 0)
    w_k = {k: dev(v) for k, v in arrays.items()}
    w_t = dict(w_k)
    fmts_t = {}
    for n in recipes.TENSORS:
        fmts_t[n] = mix[n]
        if mix[n] == Q4K:
            rows, cols = shape.matrix_shape(n)
            w_t[n] = repack(rows, cols, w_k[n])
            fmts_t[n] = Q4KT
    assert sum(f == Q4KT for f in fmts_t.values()) == 5
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    kc0 = recipes.kv_cache_array(shape, 0, "k", pos)
    vc0 = v_to_device(recipes.kv_cache_array(shape, 0, "v", pos), shape.n_kv_heads, shape.max_ctx)
    outs = []
    for fm, w in (({n: mix[n] for n in recipes.TENSORS}, w_k), (fmts_t, w_t)):
        lw = tg.layer_weights([fm[n] for n in recipes.TENSORS], [w[n] for n in recipes.TENSORS], w["attn_norm"],
                              w["ffn_norm"])
        h, kc, vc = dev(recipes.hidden_input(shape.dim)), dev(kc0), dev(vc0)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        nt.nt_decode_layer(lw, shp, pos, h.data_ptr(), kc.data_ptr(), vc.data_ptr(), ws.data_ptr(), wsb, stream())
        torch.cuda.synchronize()
        outs.append([host(h).view(np.uint32).copy(), host(kc).copy(), host(vc).copy(), host(ws).copy()])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("n_tok", [2, 5])
def test_decode_layer_k_tiled(n_tok):
    """The k-token layer (the verification pass) over tiled Q4_K matrices: the k-token GEMM runs
    on the vector units for Q4_KT at every k, so with two tokens (vector units for Q4_K too) the
    outputs are bit for bit those of the Q4_K weights, and with five (matrix cores for Q4_K)
    they agree to rounding."""
    shape, pos = SMALL, 40
    say(f"k-token layer Q4_K_M with tiled Q4_K, k={n_tok}, pos={pos}")
    mix = recipes.MIX_Q4_K_M
    arrays = recipes.layer_arrays(shape, mix, 0)
    w_k = {k: dev(v) for k, v in arrays.items()}
    w_t = dict(w_k)
    fm_t = {n: mix[n] for n in recipes.TENSORS}
    for n in recipes.TENSORS:
        if mix[n] == Q4K:
            w_t[n] = repack(*shape.matrix_shape(n), w_k[n])
            fm_t[n] = Q4KT
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_k_ws_bytes(shp, n_tok)
    kc0 = recipes.kv_cache_array(shape, 0, "k", pos)
    vc0 = v_to_device(recipes.kv_cache_array(shape, 0, "v", pos), shape.n_kv_heads, shape.max_ctx)
    h0 = np.stack([recipes.hidden_input(shape.dim, seed=t) for t in range(n_tok)]).astype(np.float32)
    outs = []
    for fm, w in (({n: mix[n] for n in recipes.TENSORS}, w_k), (fm_t, w_t)):
        lw = tg.layer_weights([fm[n] for n in recipes.TENSORS], [w[n] for n in recipes.TENSORS], w["attn_norm"],
                              w["ffn_norm"])
        h, kc, vc = dev(h0), dev(kc0), dev(vc0)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        nt.nt_decode_layer_k(lw, shp, pos, n_tok, h.data_ptr(), kc.data_ptr(), vc.data_ptr(), ws.data_ptr(), wsb,
                             stream())
        torch.cuda.synchronize()
        outs.append((host(h).copy(), host(kc).copy(), host(vc).copy()))
    (h_k, kc_k, vc_k), (h_t, kc_t, vc_t) = outs
    if n_tok == 2:
        assert np.array_equal(h_k.view(np.uint32), h_t.view(np.uint32))
        assert np.array_equal(kc_k, kc_t) and np.array_equal(vc_k, vc_t)
    else:
        scale = np.abs(h_k).max()
        assert np.max(np.abs(h_k - h_t)) <= 1e-4 * scale


# ------------------------------------------------------------------ Q8_0T

Q80, Q80T = synth.Q8_0, synth.Q8_0T


def q8t_layout(blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The NT_Q8_0T bytes of a Q8_0 matrix as include/nt.h describes them: per row, tiles of
    64 blocks (m in the last), the first 16 codes of each block, then the last 16, then the
    scales."""
    nb = cols // 32
    b = blocks.reshape(rows, nb, 34)
    out = np.empty((rows, nb * 34), np.uint8)
    for t0 in range(0, nb, 64):
        m = min(64, nb - t0)
        tile = b[:, t0:t0 + m]
        base = 34 * t0
        out[:, base:base + 16 * m] = tile[:, :, 2:18].reshape(rows, -1)
        out[:, base + 16 * m:base + 32 * m] = tile[:, :, 18:34].reshape(rows, -1)
        out[:, base + 32 * m:base + 34 * m] = tile[:, :, 0:2].reshape(rows, -1)
    return out.ravel()


def repack_to(fmt, rows, cols, src):
    dst = torch.empty_like(src)
    nt.nt_repack(fmt, rows, cols, src.data_ptr(), dst.data_ptr(), stream())
    return dst


@pytest.fixture
def register_path():
    """Q8_0 in GGUF order on the register path at every size (the launch policy streams large
    Q8_0 launches), so that it runs the same products as Q8_0T."""
    old = nt.nt_set_stream_min_weights(10 ** 15)
    yield
    nt.nt_set_stream_min_weights(old)


Q8_SHAPES = [(1, 256), (7, 768), (3, 4096), (5, 14336), (2, 2304), (3, 1792), (33, 4096 + 256 * 3)]


@pytest.mark.parametrize("rows,cols", Q8_SHAPES)
def test_repack_q8_0t_layout_and_dequant_bit_exact(rows, cols):
    say(f"repack Q8_0 -> Q8_0T {rows}x{cols}")
    blocks = synth.quant_matrix(Q80, rows, cols, seed=3, stream=2200)
    t = repack_to(Q80T, rows, cols, dev(blocks))
    assert np.array_equal(host(t), q8t_layout(blocks, rows, cols))
    w = torch.empty(rows * cols, dtype=torch.float32, device="cuda")
    nt.nt_dequant(Q80T, rows, cols, t.data_ptr(), w.data_ptr(), stream())
    assert same_value(host(w).reshape(rows, cols), oracle.dequant_f32(Q80, rows, cols, blocks))


# one block, partial tiles, the 8B shapes (14336 x 4096 and 28672 x 4096 from 10^8 weights:
# nontemporal loads), the widest x
Q8_GEMV_SHAPES = [(1, 256), (23, 1280), (130, 4352), (4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336),
                  (28672, 4096), (64, nt.NT_GEMV_MAX_COLS)]


@pytest.mark.parametrize("rows,cols", Q8_GEMV_SHAPES)
def test_gemv_q8_0t_matches_oracle(rows, cols):
    """Q8_0T's lanes take a tile's blocks in order where Q8_0's take even then odd blocks, so the
    sums are ordered differently and the two agree within the tolerance, not bit for bit."""
    say(f"gemv Q8_0T {rows}x{cols}")
    blocks = synth.quant_matrix(Q80, rows, cols, seed=0, stream=2300)
    x = synth.normal_f32(cols, seed=0, stream=2301)
    w, xd = dev(blocks), dev(x)
    y_t = gemv(Q80T, rows, cols, repack_to(Q80T, rows, cols, w), xd)
    ref, nrm = oracle.gemv(Q80, rows, cols, blocks, x.astype(np.float64))
    worst = check_rel(y_t, ref, nrm, what=f"Q8_0T {rows}x{cols}")
    say(f"  worst rel err {worst:.2e}")


@pytest.mark.parametrize("rows,cols,n_tok", [(1, 256, 1), (17, 512, 4), (300, 4352, 6), (40, 32768, 8),
                                             (14336, 4096, 7), (512, 6144, 2)])
def test_gemm_q8_0t_matches_oracle(rows, cols, n_tok):
    say(f"gemm Q8_0T {rows}x{cols} x {n_tok}")
    blocks = synth.quant_matrix(Q80, rows, cols, seed=8, stream=2400)
    X = np.stack([synth.normal_f32(cols, seed=8, stream=2401 + t) for t in range(n_tok)])
    w = repack_to(Q80T, rows, cols, dev(blocks))
    xd = dev(X.astype(np.float32))
    Y = torch.empty(n_tok * rows, dtype=torch.float32, device="cuda")
    nt.nt_gemm_q(Q80T, rows, cols, n_tok, w.data_ptr(), xd.data_ptr(), Y.data_ptr(), stream())
    Y = host(Y).reshape(n_tok, rows)
    ref, nrm = oracle.gemm(Q80, rows, cols, blocks, X.astype(np.float64))
    for t in range(n_tok):
        check_rel(Y[t], ref[t], nrm[t], what=f"Q8_0T {rows}x{cols} token {t}")


def test_embed_row_q8_0t_equals_q8_0():
    vocab, dim = 1000, 4352
    table = dev(synth.quant_matrix(Q80, vocab, dim, seed=4, stream=2500))
    tiled = repack_to(Q80T, vocab, dim, table)
    for tok in (0, 63, 64, vocab - 1):
        t = torch.tensor([tok], dtype=torch.int32, device="cuda")
        a = torch.empty(dim, dtype=torch.float32, device="cuda")
        b = torch.empty(dim, dtype=torch.float32, device="cuda")
        nt.nt_embed_row(Q80, vocab, dim, table.data_ptr(), t.data_ptr(), a.data_ptr(), stream())
        nt.nt_embed_row(Q80T, vocab, dim, tiled.data_ptr(), t.data_ptr(), b.data_ptr(), stream())
        assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32)), tok


@pytest.mark.parametrize("vocab,dim", [(1000, 1024), (128256, 4096)])
def test_lm_head_q8_0t_matches_oracle(vocab, dim):
    say(f"LM head Q8_0T {vocab}x{dim}")
    blocks = synth.quant_matrix(Q80, vocab, dim, seed=5, stream=2600)
    tiled = repack_to(Q80T, vocab, dim, dev(blocks))
    onorm_h = synth.uniform_f32(dim, 5, 2601, 0.9, 1.1)
    h_h = synth.normal_f32(dim, seed=5, stream=2602)
    onorm, h = dev(onorm_h), dev(h_h)
    res = []
    for fmt, w in ((Q80T, tiled),):
        logits = torch.empty(vocab, dtype=torch.float32, device="cuda")
        tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        ws = torch.zeros(nt.NT_LM_HEAD_WS_BYTES, dtype=torch.uint8, device="cuda")
        nt.nt_lm_head(fmt, vocab, dim, w.data_ptr(), onorm.data_ptr(), 1e-5, h.data_ptr(), logits.data_ptr(),
                      tok.data_ptr(), ws.data_ptr(), ws.numel(), stream())
        torch.cuda.synchronize()
        res.append((int(tok.item()), host(logits).copy()))
    tok, logits = res[0]
    ref, nrm = oracle.gemv(Q80, vocab, dim, blocks, oracle.rmsnorm(h_h, onorm_h, 1e-5))
    check_rel(logits, ref, nrm, what=f"Q8_0T head {vocab}x{dim}")
    assert tok == int(np.argmax(logits)) and ref[tok] >= ref.max() - 1e-3 * nrm[tok]


@pytest.mark.parametrize("shape,pos", [(SMALL, 5), (recipes.LLAMA3_8B, 1023)])
def test_decode_layer_q8_0t_close_to_q8_0(shape, pos, register_path):
    """The fused Q8_0 layer with every matrix tiled gives h within rounding of the Q8_0 matrices
    on the register path (the products are ordered differently; the stage-wise check against
    the checker is tests/test_gpu_model_8b.py, whose model holds its matrices tiled)."""
    say(f"decode layer Q8_0 tiled, dim={shape.dim} pos={pos}")
    mix = recipes.MIX_Q8_0
    arrays = recipes.layer_arrays(shape, mix, 0)
    w_k = {k: dev(v) for k, v in arrays.items()}
    w_t = dict(w_k)
    for n in recipes.TENSORS:
        w_t[n] = repack_to(Q80T, *shape.matrix_shape(n), w_k[n])
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    kc0 = recipes.kv_cache_array(shape, 0, "k", pos)
    vc0 = v_to_device(recipes.kv_cache_array(shape, 0, "v", pos), shape.n_kv_heads, shape.max_ctx)
    outs = []
    for f, w in ((Q80, w_k), (Q80T, w_t)):
        lw = tg.layer_weights([f] * len(recipes.TENSORS), [w[n] for n in recipes.TENSORS], w["attn_norm"],
                              w["ffn_norm"])
        h, kc, vc = dev(recipes.hidden_input(shape.dim)), dev(kc0), dev(vc0)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        nt.nt_decode_layer(lw, shp, pos, h.data_ptr(), kc.data_ptr(), vc.data_ptr(), ws.data_ptr(), wsb, stream())
        torch.cuda.synchronize()
        outs.append(host(h).copy())
    assert np.max(np.abs(outs[0] - outs[1])) <= 1e-4 * np.abs(outs[0]).max()


# ------------------------------------------------------------------ Q5_KT

Q5K, Q5KT = synth.Q5_K, synth.Q5_KT


def q5kt_layout(blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The NT_Q5_KT bytes of a Q5_K matrix as include/nt.h describes them."""
    nsb = cols // 256
    b = blocks.reshape(rows, nsb, 176)
    out = np.empty((rows, nsb * 176), np.uint8)
    for t0 in range(0, nsb, 16):
        m = min(16, nsb - t0)
        tile = b[:, t0:t0 + m]
        base = 176 * t0
        for part, (lo, hi) in enumerate(((0, 16), (16, 32), (32, 48))):
            out[:, base + 16 * m * part:base + 16 * m * (part + 1)] = tile[:, :, lo:hi].reshape(rows, -1)
        qs = tile[:, :, 48:].reshape(rows, m, 4, 2, 16)
        out[:, base + 48 * m:base + 112 * m] = qs[:, :, :, 0, :].reshape(rows, -1)
        out[:, base + 112 * m:base + 176 * m] = qs[:, :, :, 1, :].reshape(rows, -1)
    return out.ravel()


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_repack_q5_kt_layout_and_dequant_bit_exact(rows, cols):
    say(f"repack Q5_K -> Q5_KT {rows}x{cols}")
    blocks = synth.quant_matrix(Q5K, rows, cols, seed=3, stream=3200)
    t = repack_to(Q5KT, rows, cols, dev(blocks))
    assert np.array_equal(host(t), q5kt_layout(blocks, rows, cols))
    w = torch.empty(rows * cols, dtype=torch.float32, device="cuda")
    nt.nt_dequant(Q5KT, rows, cols, t.data_ptr(), w.data_ptr(), stream())
    assert same_value(host(w).reshape(rows, cols), oracle.dequant_f32(Q5K, rows, cols, blocks))


@pytest.mark.parametrize("rows,cols", GEMV_SHAPES)
def test_gemv_q5_kt_equals_q5_k_and_matches_oracle(rows, cols):
    say(f"gemv Q5_KT {rows}x{cols}")
    blocks = synth.quant_matrix(Q5K, rows, cols, seed=0, stream=3300)
    x = synth.normal_f32(cols, seed=0, stream=3301)
    w, xd = dev(blocks), dev(x)
    y_k = gemv(Q5K, rows, cols, w, xd)
    y_t = gemv(Q5KT, rows, cols, repack_to(Q5KT, rows, cols, w), xd)
    assert np.array_equal(y_t.view(np.uint32), y_k.view(np.uint32))
    ref, nrm = oracle.gemv(Q5K, rows, cols, blocks, x.astype(np.float64))
    check_rel(y_t, ref, nrm, what=f"Q5_KT {rows}x{cols}")


@pytest.mark.parametrize("rows,cols,n_tok", [(1, 256, 1), (37, 2304, 3), (300, 16640, 6), (40, 32768, 5), (512, 8192, 2)])
def test_gemm_q5_kt_matches_oracle(rows, cols, n_tok):
    say(f"gemm Q5_KT {rows}x{cols} x {n_tok}")
    blocks = synth.quant_matrix(Q5K, rows, cols, seed=8, stream=3400)
    X = np.stack([synth.normal_f32(cols, seed=8, stream=3401 + t) for t in range(n_tok)])
    w = repack_to(Q5KT, rows, cols, dev(blocks))
    xd = dev(X.astype(np.float32))
    Y = torch.empty(n_tok * rows, dtype=torch.float32, device="cuda")
    nt.nt_gemm_q(Q5KT, rows, cols, n_tok, w.data_ptr(), xd.data_ptr(), Y.data_ptr(), stream())
    Y = host(Y).reshape(n_tok, rows)
    ref, nrm = oracle.gemm(Q5K, rows, cols, blocks, X.astype(np.float64))
    for t in range(n_tok):
        check_rel(Y[t], ref[t], nrm[t], what=f"Q5_KT {rows}x{cols} token {t}")


@pytest.mark.parametrize("shape,pos", [(SMALL, 33), (recipes.LLAMA31_70B, 4096)])
def test_decode_layer_q5_kt_equals_q5_k(shape, pos):
    """The Q5_K_M layer with its Q5_K matrices tiled gives h, the new K and V and every stage in
    the workspace bit for bit as with the Q5_K ones."""
    say(f"decode layer Q5_K_M with tiled Q5_K, dim={shape.dim} pos={pos}")
    mix = recipes.MIX_Q5_K_M
    arrays = recipes.layer_arrays(shape, mix, 0)
    w_k = {k: dev(v) for k, v in arrays.items()}
    w_t = dict(w_k)
    fm_t = {n: mix[n] for n in recipes.TENSORS}
    for n in recipes.TENSORS:
        if mix[n] == Q5K:
            w_t[n] = repack_to(Q5KT, *shape.matrix_shape(n), w_k[n])
            fm_t[n] = Q5KT
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    kc0 = recipes.kv_cache_array(shape, 0, "k", pos)
    vc0 = v_to_device(recipes.kv_cache_array(shape, 0, "v", pos), shape.n_kv_heads, shape.max_ctx)
    outs = []
    for fm, w in (({n: mix[n] for n in recipes.TENSORS}, w_k), (fm_t, w_t)):
        lw = tg.layer_weights([fm[n] for n in recipes.TENSORS], [w[n] for n in recipes.TENSORS], w["attn_norm"],
                              w["ffn_norm"])
        h, kc, vc = dev(recipes.hidden_input(shape.dim)), dev(kc0), dev(vc0)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        nt.nt_decode_layer(lw, shp, pos, h.data_ptr(), kc.data_ptr(), vc.data_ptr(), ws.data_ptr(), wsb, stream())
        torch.cuda.synchronize()
        outs.append([host(h).view(np.uint32).copy(), host(kc).copy(), host(vc).copy(), host(ws).copy()])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
