"""The seeded input generator: reproducible, regenerable per row/slot, and with
the field distributions the workloads ask for (CPU only)."""
from __future__ import annotations

import numpy as np

import oracle
import synth
from synth import recipes


def test_reproducible_and_stream_separated():
    a = synth.quant_matrix(synth.Q4_K, 8, 512, seed=0, stream=1)
    b = synth.quant_matrix(synth.Q4_K, 8, 512, seed=0, stream=1)
    c = synth.quant_matrix(synth.Q4_K, 8, 512, seed=0, stream=2)
    d = synth.quant_matrix(synth.Q4_K, 8, 512, seed=1, stream=1)
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)


def test_rows_regenerate_alone():
    for fmt in (synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q5_K):
        full = synth.quant_matrix(fmt, 12, 1024, seed=0, stream=9).reshape(12, -1)
        part = synth.quant_rows(fmt, 1024, [11, 0, 5], seed=0, stream=9)
        assert np.array_equal(part, full[[11, 0, 5]])


def test_q8_0_fields():
    blk = synth.quant_matrix(synth.Q8_0, 64, 4096, seed=0, stream=3).reshape(-1, 34)
    d = blk[:, :2].copy().view(np.float16).astype(np.float64).ravel()
    q = blk[:, 2:].view(np.int8)
    assert d.min() >= 0.001 - 1e-6 and d.max() <= 0.01 + 1e-5
    assert q.min() == -127 and q.max() == 127
    assert abs(q.mean()) < 0.5
    counts = np.bincount(q.ravel().astype(np.int64) + 127, minlength=255)
    assert counts.min() > 0.8 * counts.mean()


def test_q4_k_and_q6_k_fields_uniform():
    blk = synth.quant_matrix(synth.Q4_K, 64, 8192, seed=0, stream=4).reshape(-1, 144)
    d = blk[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    dmin = blk[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    assert 0.0009 < d.min() and d.max() < 0.0101 and 0.0009 < dmin.min() and dmin.max() < 0.0101
    nib = np.concatenate([blk[:, 16:] & 15, blk[:, 16:] >> 4]).ravel()
    cnt = np.bincount(nib, minlength=16)
    assert cnt.min() > 0.95 * cnt.mean()
    q6 = synth.quant_matrix(synth.Q6_K, 64, 8192, seed=0, stream=5).reshape(-1, 210)
    s = q6[:, 192:208].view(np.int8)
    assert s.min() == -64 and s.max() == 63
    d6 = q6[:, 208:210].copy().view(np.float16).astype(np.float64).ravel()
    assert 0.0009 < d6.min() and d6.max() < 0.0101
    # decoded codes are uniform over 0..63 (decode through the checker)
    w = oracle.dequant_exact(synth.Q6_K, 4, 8192, q6[:4 * 32].ravel())
    assert np.isfinite(w).all()


def test_q5_k_fields_uniform():
    blk = synth.quant_matrix(synth.Q5_K, 64, 8192, seed=0, stream=11).reshape(-1, 176)
    d = blk[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    dmin = blk[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    assert 0.0009 < d.min() and d.max() < 0.0101 and 0.0009 < dmin.min() and dmin.max() < 0.0101
    bits = np.unpackbits(blk[:, 16:48].ravel())
    assert abs(bits.mean() - 0.5) < 0.01
    nib = np.concatenate([blk[:, 48:] & 15, blk[:, 48:] >> 4]).ravel()
    cnt = np.bincount(nib, minlength=16)
    assert cnt.min() > 0.95 * cnt.mean()


def test_normals_and_gains():
    x = synth.normal_f32(200000, seed=0, stream=6)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    g = synth.uniform_f32(100000, seed=0, stream=7, lo=0.9, hi=1.1)
    assert g.min() >= 0.9 and g.max() <= 1.1 and abs(g.mean() - 1.0) < 0.001
    h = synth.normal_f16_bits(100000, seed=0, stream=8).view(np.float16).astype(np.float64)
    assert abs(h.std() - 1) < 0.02
    # element offsets address the same stream
    assert np.array_equal(synth.normal_f32(10, 0, 6, e0=5), x[5:15])


def test_kv_cache_slots_and_layout():
    shp = recipes.LayerShape(dim=256, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn_dim=256, max_ctx=6)
    kc = recipes.kv_cache_array(shp, 3, "k", 4)
    assert np.all(kc[:, 4:] == 0) and np.all(kc[:, :4] != 0)
    full = recipes.kv_cache_array(shp, 3, "k", 6)
    assert np.array_equal(full[:, :4], kc[:, :4])


def test_blob_layout_aligned_and_disjoint():
    for shp, mix in ((recipes.LLAMA31_70B, recipes.MIX_Q4_K_M), (recipes.LLAMA31_70B, recipes.MIX_Q6_K),
                     (recipes.LLAMA3_8B, recipes.MIX_Q8_0)):
        lay = recipes.blob_layout(shp, mix)
        offs = lay.offset_list()
        assert all(o % 256 == 0 for o in offs)
        assert offs == sorted(offs) and lay.nbytes >= offs[-1] + 4 * shp.dim
    assert recipes.blob_layout(recipes.LLAMA31_70B, recipes.MIX_Q6_K).nbytes >= 701_890_560
