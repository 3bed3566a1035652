"""GPU parity of the per-op C ABI against the fp64 checker (MI355X only).

Every call goes through libnt.so's C ABI.  Acceptance: dequantization bit-exact
(by value); GEMV |y - y_ref| <= 1e-3 * sum_c |w_rc x_c| per row (and exactly 0
where that sum is 0); the small ops within 1e-3 of their own normalisers.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import quantized_weight_streaming_dequant_amd as nt
import synth
from synth import recipes
from tests.blockpack import pack_q4_0, pack_q4_k, pack_q5_k, pack_q6_k, pack_q8_0
from tests.gpu_util import v_to_device, check_rel, dev, host, same_value, say, stream

pytestmark = pytest.mark.gpu

FMTS = [synth.Q8_0, synth.Q4_0, synth.Q4_K, synth.Q6_K, synth.Q5_K, synth.F16, synth.F32]
NAMES = synth.FORMAT_NAMES


def gpu_gemv(fmt, rows, cols, blocks, x):
    wb = dev(blocks)
    xd = dev(x.astype(np.float32))
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    nt.nt_gemv_q(fmt, rows, cols, wb.data_ptr(), xd.data_ptr(), y.data_ptr(), stream())
    return host(y)


def gpu_dequant(fmt, rows, cols, blocks):
    wb = dev(blocks)
    w = torch.empty(rows * cols, dtype=torch.float32, device="cuda")
    nt.nt_dequant(fmt, rows, cols, wb.data_ptr(), w.data_ptr(), stream())
    return host(w).reshape(rows, cols)


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1, 256), (7, 768), (33, 4096), (5, 28672)])
def test_dequant_bit_exact(fmt, rows, cols):
    say(f"dequant {NAMES[fmt]} {rows}x{cols}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=1, stream=100 + fmt)
    got = gpu_dequant(fmt, rows, cols, blocks)
    ref = oracle.dequant_f32(fmt, rows, cols, blocks)
    assert same_value(got, ref)


def test_dequant_hand_blocks_bit_exact():
    say("dequant hand blocks")
    cases = [
        (synth.Q8_0, pack_q8_0(-3.0, [-128, 127] * 16) + pack_q8_0(2.0 ** -24, list(range(-16, 16)))),
        (synth.Q4_0, pack_q4_0(65504.0, list(range(16)) * 2) + pack_q4_0(-0.5, [15 - (i % 16) for i in range(32)])),
        (synth.Q4_K, pack_q4_k(0.001, 0.01, [63] * 8, [63] * 8, [i % 16 for i in range(256)]) +
         pack_q4_k(-2.0, 6.1e-5, list(range(56, 64)), list(range(8)), [(i * 7) % 16 for i in range(256)])),
        (synth.Q6_K, pack_q6_k(0.01, [-128, 127] * 8, [i % 64 for i in range(256)]) +
         pack_q6_k(-6.0e-8, [-64 + 8 * k for k in range(16)], [(i * 5 + 3) % 64 for i in range(256)])),
        (synth.Q5_K, pack_q5_k(0.001, 0.01, [63] * 8, [63] * 8, [i % 32 for i in range(256)]) +
         pack_q5_k(-2.0, 6.1e-5, list(range(56, 64)), list(range(8)), [(i * 7 + 16 * (i // 32 % 2)) % 32
                                                                      for i in range(256)])),
    ]
    # F16 / F32: the IEEE values themselves, specials included
    f16 = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0x3C00, 0xC000, 0xFBFF, 0x3555] * 6 + [0x1234] * 4,
                   dtype=np.uint16)
    f32 = np.array([0.0, -0.0, 1.401298464324817e-45, 3.4028234663852886e38, -1.0, 0.1, -2.5e-30, 65504.0] * 8,
                   dtype=np.float32)
    cases += [(synth.F16, f16.tobytes()), (synth.F32, f32.tobytes())]
    for fmt, raw in cases:
        blocks = np.frombuffer(raw, np.uint8)
        cols = synth.BLOCK_ELEMS[fmt] * 2 if synth.BLOCK_ELEMS[fmt] > 1 else len(raw) // synth.BLOCK_BYTES[fmt]
        got = gpu_dequant(fmt, 1, cols, blocks)
        ref = oracle.dequant_f32(fmt, 1, cols, blocks)
        assert same_value(got, ref), NAMES[fmt]


def test_dequant_f16_every_code():
    """All 65536 binary16 codes as one F16 matrix: each dequantizes to its value (NaN as NaN)."""
    codes = np.arange(65536, dtype=np.uint16)
    got = gpu_dequant(synth.F16, 64, 1024, codes.view(np.uint8))
    ref = oracle.dequant_f32(synth.F16, 64, 1024, codes.view(np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and same_value(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------------------ GEMV

GEMV_SHAPES = {
    # rows x cols: single block, ragged block counts (odd row byte counts put rows at
    # alternating 4-byte phases: the register path), rows past a workgroup's task range,
    # 16-byte-aligned rows with a partial last column slice (the streamed path), and the
    # workload shapes
    synth.Q8_0: [(1, 32), (3, 32), (37, 2144), (301, 1056), (37, 2304), (3, 256), (4096, 4096), (14336, 4096),
                 (4096, 14336)],
    synth.Q4_0: [(1, 32), (5, 96), (29, 1440), (29, 2304), (257, 4096), (4096, 4096)],
    synth.Q4_K: [(1, 256), (23, 1280), (130, 4352), (3, 12288), (8192, 8192), (1024, 8192), (28672, 8192),
                 (8192, 28672)],
    synth.Q6_K: [(1, 256), (19, 768), (77, 2304), (77, 6144), (5, 2048), (8192, 8192), (1024, 8192), (28672, 8192),
                 (8192, 28672)],
    synth.Q5_K: [(1, 256), (23, 1280), (130, 4352), (3, 12288), (8192, 8192), (1024, 8192), (28672, 8192),
                 (8192, 28672)],
    # unquantized: one 32-column unit, a last step of one unit (2080 = 2048 + 32 for F16, 1024 + 1024 + 32
    # for F32), the workload shapes
    synth.F16: [(1, 32), (3, 96), (37, 2080), (130, 4352), (8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)],
    synth.F32: [(1, 32), (3, 96), (37, 2080), (130, 4352), (8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)],
}
GEMV_CASES = [(f, r, c) for f in FMTS for (r, c) in GEMV_SHAPES[f]]
# the widest x the header allows (NT_GEMV_MAX_COLS columns)
GEMV_CASES += [(f, 64, nt.NT_GEMV_MAX_COLS) for f in FMTS]


@pytest.mark.parametrize("fmt,rows,cols", GEMV_CASES)
def test_gemv_matches_oracle(fmt, rows, cols):
    say(f"gemv {NAMES[fmt]} {rows}x{cols}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=0, stream=200 + fmt)
    x = synth.normal_f32(cols, seed=0, stream=300 + fmt)
    y = gpu_gemv(fmt, rows, cols, blocks, x)
    ref, nrm = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
    worst = check_rel(y, ref, nrm, what=f"{NAMES[fmt]} {rows}x{cols}")
    say(f"  worst rel err {worst:.2e}")


# The streamed path at the shapes built for its edge cases (rows past a workgroup's task
# range, a partial last column slice, single blocks): the launch policy sends launches under
# 10^8 weights to the register path, so these force it with a threshold of 0.
STREAMED_CASES = [(f, r, c) for f in (synth.Q8_0, synth.Q4_0, synth.Q6_K) for (r, c) in GEMV_SHAPES[f]
                  if r * c < 10 ** 8] + [(f, 64, nt.NT_GEMV_MAX_COLS) for f in (synth.Q8_0, synth.Q4_0, synth.Q6_K)]


@pytest.fixture
def streamed_path():
    prev = nt.nt_set_stream_min_weights(0)
    yield
    nt.nt_set_stream_min_weights(prev)


@pytest.mark.parametrize("fmt,rows,cols", STREAMED_CASES)
def test_gemv_streamed_path_matches_oracle(fmt, rows, cols, streamed_path):
    say(f"gemv (streamed path) {NAMES[fmt]} {rows}x{cols}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=0, stream=200 + fmt)
    x = synth.normal_f32(cols, seed=0, stream=300 + fmt)
    y = gpu_gemv(fmt, rows, cols, blocks, x)
    ref, nrm = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
    worst = check_rel(y, ref, nrm, what=f"{NAMES[fmt]} {rows}x{cols}")
    say(f"  worst rel err {worst:.2e}")


# The register path at the workload shapes the launch policy streams (10^8 weights and up,
# or from 1.25 10^7 where each register-path wave would run 7 or more items in a row): a
# threshold no launch reaches keeps them on the register path.
REGISTER_CASES = [(synth.Q8_0, 4096, 14336), (synth.Q8_0, 14336, 4096), (synth.Q6_K, 28672, 8192),
                  (synth.Q6_K, 8192, 28672)]


@pytest.fixture
def register_path():
    prev = nt.nt_set_stream_min_weights(1 << 62)
    yield
    nt.nt_set_stream_min_weights(prev)


@pytest.mark.parametrize("fmt,rows,cols", REGISTER_CASES)
def test_gemv_register_path_matches_oracle(fmt, rows, cols, register_path):
    say(f"gemv (register path) {NAMES[fmt]} {rows}x{cols}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=0, stream=200 + fmt)
    x = synth.normal_f32(cols, seed=0, stream=300 + fmt)
    y = gpu_gemv(fmt, rows, cols, blocks, x)
    ref, nrm = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
    worst = check_rel(y, ref, nrm, what=f"{NAMES[fmt]} {rows}x{cols}")
    say(f"  worst rel err {worst:.2e}")


def gpu_gemm(fmt, rows, cols, n_tok, blocks, X):
    wb = dev(blocks)
    xd = dev(np.ascontiguousarray(X, dtype=np.float32).ravel())
    y = torch.full((n_tok * rows,), float("nan"), dtype=torch.float32, device="cuda")
    nt.nt_gemm_q(fmt, rows, cols, n_tok, wb.data_ptr(), xd.data_ptr(), y.data_ptr(), stream())
    return host(y).reshape(n_tok, rows)


GEMM_CASES = [
    # (format, rows, cols, tokens): single blocks, ragged row counts, token counts that fill
    # the kernels' 1/2/4/8-token variants partly, the 70B shapes, and widths that run as
    # several column chunks (each adding into y)
    (synth.Q8_0, 1, 32, 8), (synth.Q8_0, 37, 2144, 3), (synth.Q8_0, 4096, 14336, 5), (synth.Q4_0, 29, 1440, 6),
    (synth.Q4_K, 1, 256, 1), (synth.Q4_K, 130, 4352, 2), (synth.Q4_K, 8192, 8192, 4), (synth.Q4_K, 1024, 8192, 8),
    (synth.Q4_K, 28672, 8192, 4), (synth.Q4_K, 8192, 28672, 7),
    (synth.Q6_K, 77, 2304, 7), (synth.Q6_K, 8192, 28672, 8), (synth.Q6_K, 1024, 8192, 3),
    (synth.Q5_K, 23, 1280, 6), (synth.Q5_K, 8192, 8192, 8), (synth.Q5_K, 28672, 8192, 2),
    # the matrix-core path (Q4_K, 3 to 8 tokens): 16-row tiles cut short, chunks of fewer
    # superblocks than waves, a one-superblock last chunk, one row
    (synth.Q4_K, 37, 2304, 3), (synth.Q4_K, 17, 512, 4), (synth.Q4_K, 1, 256, 8), (synth.Q4_K, 130, 4352, 5),
    (synth.Q4_K, 300, 16640, 6), (synth.Q4_K, 1000, 12288, 8),
    # Q6_K on the matrix cores: odd superblock counts (chunks that start 2 bytes past a
    # 4-byte boundary), one row, a short tile
    (synth.Q6_K, 17, 512, 4), (synth.Q6_K, 1, 256, 8), (synth.Q6_K, 130, 4352, 6), (synth.Q6_K, 300, 16640, 5),
    # the widest x the header allows: many column chunks adding into y
    (synth.Q4_K, 40, 32768, 8), (synth.Q6_K, 40, 32768, 4), (synth.Q8_0, 40, 32768, 3),
    # Q5_K on the matrix cores: short tiles, one row, chunks of fewer superblocks than waves, the widest x
    (synth.Q5_K, 37, 2304, 3), (synth.Q5_K, 1, 256, 8), (synth.Q5_K, 300, 16640, 6), (synth.Q5_K, 40, 32768, 5),
    # Q8_0 at 3-8 tokens (the VALU kernel: its matrix-core form measured slower), the 8B FFN shape
    (synth.Q8_0, 17, 512, 4), (synth.Q8_0, 1, 256, 8), (synth.Q8_0, 300, 4352, 6), (synth.Q8_0, 14336, 4096, 7),
    # F16 / F32 (vector ALUs, fp32 x staged per token): ragged last steps, the 70B shape, several chunks
    (synth.F16, 1, 32, 8), (synth.F16, 37, 2080, 3), (synth.F16, 8192, 8192, 4), (synth.F16, 40, 32768, 5),
    (synth.F32, 3, 96, 2), (synth.F32, 130, 4352, 5), (synth.F32, 1024, 8192, 8), (synth.F32, 40, 32768, 7),
]


@pytest.mark.parametrize("fmt,rows,cols,n_tok", GEMM_CASES)
def test_gemm_matches_oracle(fmt, rows, cols, n_tok):
    say(f"gemm {NAMES[fmt]} {rows}x{cols} x {n_tok} tokens")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=8, stream=700 + fmt)
    X = np.stack([synth.normal_f32(cols, seed=8, stream=800 + t) for t in range(n_tok)])
    Y = gpu_gemm(fmt, rows, cols, n_tok, blocks, X)
    ref, nrm = oracle.gemm(fmt, rows, cols, blocks, X.astype(np.float64))
    worst = 0.0
    for t in range(n_tok):
        worst = max(worst, check_rel(Y[t], ref[t], nrm[t], what=f"{NAMES[fmt]} {rows}x{cols} token {t}"))
    say(f"  worst rel err {worst:.2e}")


def test_gemm_one_token_matches_gemv_and_tokens_are_independent():
    """A token's outputs do not depend on the other tokens of the call, and one token gives
    what the GEMV gives (both are within the tolerance of the same exact values)."""
    fmt, rows, cols = synth.Q4_K, 512, 8192
    blocks = synth.quant_matrix(fmt, rows, cols, seed=9, stream=900)
    X = np.stack([synth.normal_f32(cols, seed=9, stream=901 + t) for t in range(8)])
    Xo = np.stack([synth.normal_f32(cols, seed=9, stream=951 + t) for t in range(8)])
    # token 2 kept, every other token replaced: its outputs are bit for bit the same, on the
    # VALU kernel (2 tokens) and on the matrix-core kernel (4 and 8 token slots)
    for n in (3, 4, 5, 8):
        Xb = Xo[:n].copy()
        Xb[2] = X[2]
        Ya = gpu_gemm(fmt, rows, cols, n, blocks, X[:n])
        Yb = gpu_gemm(fmt, rows, cols, n, blocks, Xb)
        assert np.array_equal(Ya[2], Yb[2]), f"{n} tokens"
    Y2 = gpu_gemm(fmt, rows, cols, 2, blocks, X[:2])
    Y2b = gpu_gemm(fmt, rows, cols, 2, blocks, np.stack([X[0], Xo[1]]))
    assert np.array_equal(Y2[0], Y2b[0])
    Y4 = gpu_gemm(fmt, rows, cols, 4, blocks, X[:4])
    y1 = gpu_gemv(fmt, rows, cols, blocks, X[1])
    ref, nrm = oracle.gemv(fmt, rows, cols, blocks, X[1].astype(np.float64))
    check_rel(y1, ref, nrm, what="gemv")
    check_rel(Y4[1], ref, nrm, what="gemm token 1")


OUTLIER_KINDS = {
    # multiplier per column on top of N(0, 1): one channel per 32 columns at 100x, a single
    # channel at 10^4x, three channels at 2000x (the shapes of large outlier activations)
    "every_block_100x": lambda c: np.where(np.arange(c) % 32 == 7, 100.0, 1.0),
    "one_channel_1e4x": lambda c: np.where(np.arange(c) == 100, 1e4, 1.0),
    "three_channels_2000x": lambda c: np.where(np.isin(np.arange(c), [100, 2000, 5000]), 2000.0, 1.0),
}


@pytest.mark.parametrize("kind", list(OUTLIER_KINDS))
@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_outlier_activations(fmt, kind):
    """x with large outlier channels: each 32-column block of x is staged on the scale of its
    largest entry, so the other entries of an outlier's block lose the most; they stay far
    inside the tolerance (worst seen ~2e-6 of sum |w x|, checked against 1e-5)."""
    rows, cols = 512, 8192
    say(f"gemv outliers {kind} {NAMES[fmt]}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=3, stream=500 + fmt)
    x = (synth.normal_f32(cols, seed=3, stream=600 + fmt) * OUTLIER_KINDS[kind](cols)).astype(np.float32)
    y = gpu_gemv(fmt, rows, cols, blocks, x)
    ref, nrm = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
    worst = check_rel(y, ref, nrm, what=f"{NAMES[fmt]} {kind}")
    if fmt not in (synth.F16, synth.F32):  # the unquantized formats read x in fp32, not as limbs
        worst = check_rel(y, ref, nrm, tol=1e-5, what=f"{NAMES[fmt]} {kind} (limb precision)")
    say(f"  worst rel err {worst:.2e}")


@pytest.mark.parametrize("mean", [50.0, -3.0])
@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_offset_activations(fmt, mean):
    """x = mean + N(0, 1): each block's sum of x is large next to the spread of x, which is
    what the kernels scale and subtract where they restore a bias from that sum (the Q4_K
    high nibbles taken as the bytes 16 n - 128, the Q4_0 codes' offset of 8, the K formats'
    minimum terms).  Held to the same limb-precision bound as the outliers."""
    rows, cols = 512, 8192
    say(f"gemv offset x mean {mean} {NAMES[fmt]}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=5, stream=510 + fmt)
    x = synth.normal_f32(cols, seed=5, stream=610 + fmt, mean=mean)
    y = gpu_gemv(fmt, rows, cols, blocks, x)
    ref, nrm = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
    worst = check_rel(y, ref, nrm, what=f"{NAMES[fmt]} mean {mean}")
    if fmt not in (synth.F16, synth.F32):
        worst = check_rel(y, ref, nrm, tol=1e-5, what=f"{NAMES[fmt]} mean {mean} (limb precision)")
    say(f"  worst rel err {worst:.2e}")


@pytest.mark.parametrize("fmt", [synth.Q4_K, synth.Q5_K, synth.Q6_K, synth.Q8_0])
@pytest.mark.parametrize("kind", list(OUTLIER_KINDS))
def test_gemm_outlier_activations(kind, fmt):
    """The same outlier channels in every token of the matrix-core GEMM (5 tokens, one token
    without outliers): the digits are the GEMV's, so the same 1e-5 bound holds."""
    rows, cols, n = 512, 8192, 5
    say(f"gemm outliers {kind}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=4, stream=520 + fmt)
    X = np.stack([synth.normal_f32(cols, seed=4, stream=620 + t) * (OUTLIER_KINDS[kind](cols) if t != 3 else 1.0)
                  for t in range(n)]).astype(np.float32)
    Y = gpu_gemm(fmt, rows, cols, n, blocks, X)
    ref, nrm = oracle.gemm(fmt, rows, cols, blocks, X.astype(np.float64))
    for t in range(n):
        check_rel(Y[t], ref[t], nrm[t], tol=1e-5, what=f"{kind} token {t} (limb precision)")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_non_finite_activation(fmt, bad):
    """One NaN or inf in x: the exact result of every row is non-finite (a nonzero weight times
    inf, or zero times inf), and so is the kernel's (the 32-column block holding it is staged with
    a NaN scale)."""
    rows, cols = 96, 2048
    blocks = synth.quant_matrix(fmt, rows, cols, seed=6, stream=540 + fmt)
    x = synth.normal_f32(cols, seed=6, stream=640 + fmt).copy()
    x[777] = bad
    ref, _ = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
    assert not np.isfinite(ref).any()
    y = gpu_gemv(fmt, rows, cols, blocks, x)
    assert not np.isfinite(y).any()


@pytest.mark.parametrize("fmt,n_tok", [(synth.Q4_K, 4), (synth.Q4_K, 7), (synth.Q6_K, 5), (synth.Q5_K, 8), (synth.Q4_K, 2),
                                       (synth.Q8_0, 3)])
def test_gemm_non_finite_token_is_isolated(fmt, n_tok):
    """A NaN in one token's x makes that token's outputs non-finite and leaves every other
    token's outputs bit for bit as without it (the matrix-core kernel puts four tokens' digits
    in one MFMA operand; each output row still meets one token's digits and scales only)."""
    rows, cols = 130, 4096
    blocks = synth.quant_matrix(fmt, rows, cols, seed=7, stream=560 + fmt)
    X = np.stack([synth.normal_f32(cols, seed=7, stream=660 + t) for t in range(n_tok)])
    Y = gpu_gemm(fmt, rows, cols, n_tok, blocks, X)
    Xb = X.copy()
    Xb[1, 1000] = float("nan")
    Yb = gpu_gemm(fmt, rows, cols, n_tok, blocks, Xb)
    assert not np.isfinite(Yb[1]).any()
    for t in range(n_tok):
        if t != 1:
            assert np.array_equal(Y[t], Yb[t]), f"token {t}"


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_one_hot_and_zero(fmt):
    """One-hot x picks a dequantized column exactly; all-zero blocks give exact zeros."""
    rows, cols = 64, 1024
    say(f"gemv one-hot {NAMES[fmt]}")
    blocks = synth.quant_matrix(fmt, rows, cols, seed=2, stream=400 + fmt)
    w32 = oracle.dequant_f32(fmt, rows, cols, blocks)
    for j in (0, 31, 32, 255, 256, 777, 1023):
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        y = gpu_gemv(fmt, rows, cols, blocks, x)
        ref, nrm = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
        check_rel(y, ref, nrm, what=f"one-hot {j}")
        # one nonzero product per row: every partial term is exact, so the only
        # rounding is the one that also makes the dequantized weight
        assert same_value(y, w32[:, j])
    zb = np.zeros_like(blocks)
    y = gpu_gemv(fmt, rows, cols, zb, synth.normal_f32(cols, 0, 5))
    assert np.all(y == 0)


def test_gemv_misaligned_base_rejected():
    blocks = dev(synth.quant_matrix(synth.Q4_K, 4, 256, 0, 1))
    x = torch.zeros(256, dtype=torch.float32, device="cuda")
    y = torch.zeros(4, dtype=torch.float32, device="cuda")
    with pytest.raises(nt.NtError) as ei:
        nt.nt_gemv_q(synth.Q4_K, 3, 256, blocks.data_ptr() + 4, x.data_ptr(), y.data_ptr(), stream())
    assert ei.value.code == nt.NT_EALIGN


# ------------------------------------------------------------------ small ops

def test_rmsnorm():
    for n in (1, 100, 4096, 8192, 28672):
        say(f"rmsnorm n={n}")
        x = synth.normal_f32(n, 0, 11) * 3.0
        g = synth.uniform_f32(n, 0, 12, 0.9, 1.1)
        xd, gd = dev(x), dev(g)
        y = torch.empty(n, dtype=torch.float32, device="cuda")
        nt.nt_rmsnorm(n, xd.data_ptr(), gd.data_ptr(), 1e-5, y.data_ptr(), stream())
        ref = oracle.rmsnorm(x, g, 1e-5)
        check_rel(host(y), ref, np.abs(ref) + 1e-30, what=f"rmsnorm {n}")


def test_rmsnorm_in_place():
    n = 8192
    x = synth.normal_f32(n, 0, 13)
    g = synth.uniform_f32(n, 0, 14, 0.9, 1.1)
    xd, gd = dev(x), dev(g)
    nt.nt_rmsnorm(n, xd.data_ptr(), gd.data_ptr(), 1e-5, xd.data_ptr(), stream())
    ref = oracle.rmsnorm(x, g, 1e-5)
    check_rel(host(xd), ref, np.abs(ref) + 1e-30)


@pytest.mark.parametrize("pos", [0, 1, 1023, 4096, 4223])
def test_rope(pos):
    say(f"rope pos={pos}")
    n_heads, hd = 72, 128
    x = synth.normal_f32(n_heads * hd, 0, 15) * 20
    xd = dev(x)
    nt.nt_rope(n_heads, hd, pos, 500000.0, xd.data_ptr(), stream())
    ref = oracle.rope(x, n_heads, hd, pos, 500000.0)
    pair = np.repeat(np.hypot(x[0::2].astype(np.float64), x[1::2]), 2)
    check_rel(host(xd), ref, pair, what=f"rope {pos}")


def test_swiglu():
    n = 28672
    g = synth.normal_f32(n, 0, 16) * 6
    g[:4] = [0.0, 100.0, -100.0, -1000.0]
    u = synth.normal_f32(n, 0, 17)
    gd, ud = dev(g), dev(u)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    nt.nt_swiglu(n, gd.data_ptr(), ud.data_ptr(), out.data_ptr(), stream())
    ref, nrm = oracle.swiglu(g, u)
    got = host(out)
    assert np.all(np.isfinite(got))
    check_rel(got, ref, nrm, what="swiglu")


ATTN_CASES = [  # n_q, n_kv, n_ctx, max_ctx, q scale
    (32, 8, 1024, 1024, 1.0), (32, 8, 1024, 1024, 8.0), (64, 8, 4097, 4224, 1.0), (64, 8, 4224, 4224, 6.0),
    (64, 8, 1, 4224, 1.0), (64, 8, 65, 128, 1.0), (64, 8, 128, 128, 1.0), (64, 8, 129, 136, 1.0),
    (8, 8, 300, 512, 1.0), (16, 8, 77, 96, 2.0), (16, 1, 333, 400, 1.0), (128, 8, 1000, 1024, 1.0),
    (64, 8, 16384, 16384, 1.0), (64, 8, 9001, 16384, 1e-6), (64, 8, 2049, 2560, 30.0),
    (8, 1, nt.NT_MAX_CTX, nt.NT_MAX_CTX, 1.0),  # the longest cache the header allows
    # the 256-slot split boundaries: one full split (one kernel), one slot into a second, two full
    (64, 8, 256, 256, 1.0), (64, 8, 257, 264, 1.0), (32, 8, 512, 512, 3.0), (16, 2, 255, 256, 1.0),
    # a few splits with a ragged last one (the 8B shape's context length and either side of it)
    (32, 8, 777, 1024, 1.0), (64, 8, 513, 520, 2.0), (8, 2, 1023, 1024, 1.0),
]


def run_attention(n_q, n_kv, n_ctx, max_ctx, q, kc, vc, reps=2):
    hd = 128
    qd, kd = dev(q), dev(kc)
    vd = dev(v_to_device(vc, n_kv, max_ctx))
    out = torch.empty(n_q * hd, dtype=torch.float32, device="cuda")
    wsb = nt.nt_attn_decode_ws_bytes(n_q, n_kv, hd, max_ctx)
    ws = torch.full((wsb,), 0xFF, dtype=torch.uint8, device="cuda")  # no initial contents are needed
    res = []
    for rep in range(reps):
        nt.nt_attn_decode(n_q, n_kv, hd, n_ctx, max_ctx, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(),
                          ws.data_ptr(), wsb, stream())
        res.append(host(out).copy())
    return res


@pytest.mark.parametrize("n_q,n_kv,n_ctx,max_ctx,qs", ATTN_CASES)
def test_attention(n_q, n_kv, n_ctx, max_ctx, qs):
    say(f"attention nq={n_q} nkv={n_kv} n_ctx={n_ctx} max_ctx={max_ctx} qscale={qs}")
    hd = 128
    q = synth.normal_f32(n_q * hd, 0, 18) * qs
    kc = synth.normal_f16_bits(n_kv * max_ctx * hd, 0, 19)
    vc = synth.normal_f16_bits(n_kv * max_ctx * hd, 0, 20)
    ref, nrm = oracle.attn(q, kc, vc, n_q, n_kv, hd, n_ctx, max_ctx)
    outs = run_attention(n_q, n_kv, n_ctx, max_ctx, q, kc, vc)
    for rep, got in enumerate(outs):
        check_rel(got, ref, nrm, what=f"attention rep {rep}")
    assert same_value(outs[0], outs[1])  # no state carried between calls


@pytest.mark.parametrize("n_ctx", [1, 37, 131, 1000])
def test_attention_ignores_slots_past_n_ctx(n_ctx):
    """Slots at or past n_ctx may hold any bits (here NaN and inf) without affecting the result."""
    n_q, n_kv, max_ctx, hd = 64, 8, 1024, 128
    say(f"attention with NaN/inf past n_ctx={n_ctx}")
    q = synth.normal_f32(n_q * hd, 0, 22)
    kc = synth.normal_f16_bits(n_kv * max_ctx * hd, 0, 23).reshape(n_kv, max_ctx, hd)
    vc = synth.normal_f16_bits(n_kv * max_ctx * hd, 0, 24).reshape(n_kv, max_ctx, hd)
    kc[:, n_ctx:, 0::2] = 0x7E00  # NaN
    kc[:, n_ctx:, 1::2] = 0x7C00  # +inf
    vc[:, n_ctx:, 0::2] = 0xFC00  # -inf
    vc[:, n_ctx:, 1::2] = 0x7E00
    ref, nrm = oracle.attn(q, kc.ravel(), vc.ravel(), n_q, n_kv, hd, n_ctx, max_ctx)
    (got,) = run_attention(n_q, n_kv, n_ctx, max_ctx, q, kc.ravel(), vc.ravel(), reps=1)
    check_rel(got, ref, nrm, what="attention")


def test_attention_one_hot_is_exact_value_row():
    """A query that selects one slot by a huge margin returns that slot's V row (fp16 values,
    exactly representable): the split merge and the hi/lo products must not disturb it."""
    n_q, n_kv, max_ctx, n_ctx, hd = 16, 2, 1024, 700, 128
    say("attention one-hot")
    kc = np.zeros((n_kv, max_ctx, hd), np.uint16)
    vc = synth.normal_f16_bits(n_kv * max_ctx * hd, 0, 25).reshape(n_kv, max_ctx, hd)
    pick = [5, 311, 698, 0, 130, 129, 127, 640]  # slot per query head of group 0; group 1 mirrors it
    kc[:, :, :] = np.float16(0.0).view(np.uint16)
    q = np.zeros((n_q, hd), np.float32)
    for h in range(n_q):
        g = h // (n_q // n_kv)
        t = pick[h % 8]
        kc[g, t, h % 8] = np.float16(1.0).view(np.uint16)
        q[h, h % 8] = 4000.0  # score 4000/sqrt(128) ~ 354 above every other slot
    outs = run_attention(n_q, n_kv, n_ctx, max_ctx, q.ravel(), kc.ravel(), vc.ravel(), reps=1)
    got = outs[0].reshape(n_q, hd)
    vf = vc.view(np.float16).astype(np.float32)
    for h in range(n_q):
        g = h // (n_q // n_kv)
        assert np.array_equal(got[h], vf[g, pick[h % 8]]), h


# ------------------------------------------------------------------ token glue

def test_embed_row_and_argmax():
    fmt, vocab, dim = synth.Q4_K, 1000, 1024
    say("embed row + argmax")
    table = synth.quant_matrix(fmt, vocab, dim, 0, 21)
    td = dev(table)
    h = torch.empty(dim, dtype=torch.float32, device="cuda")
    for tok in (0, 1, 517, 999, -1, 1000):
        t = torch.tensor([tok], dtype=torch.int32, device="cuda")
        nt.nt_embed_row(fmt, vocab, dim, td.data_ptr(), t.data_ptr(), h.data_ptr(), stream())
        got = host(h)
        if 0 <= tok < vocab:
            assert same_value(got, oracle.dequant_f32(fmt, vocab, dim, table)[tok])
        else:
            assert np.all(got == 0)
    for n in (1, 7, 128256):
        v = synth.normal_f32(n, 0, 22)
        if n > 7:
            v[5000] = v[90000] = v.max() + 1  # a tie: the lower index wins
        vd = dev(v)
        o = torch.zeros(1, dtype=torch.int32, device="cuda")
        nt.nt_argmax(n, vd.data_ptr(), o.data_ptr(), stream())
        assert int(host(o)[0]) == oracle.argmax(v)


def test_read_probe_runs_and_leaves_the_sink():
    """The read-rate probe streams a buffer and discards it: it returns, and the sink keeps
    its value unless the folded data hits the one constant it stores on (not these bytes)."""
    n = 64 << 20
    buf = torch.zeros(n, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    nt.nt_read_probe(buf.data_ptr(), n, sink.data_ptr(), stream())
    nt.nt_read_probe(buf.data_ptr(), 16, sink.data_ptr(), stream())  # a single 16-byte piece
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


def test_gemv_from_several_host_threads():
    """Host threads on their own streams launch GEMVs of different widths (so of different LDS
    sizes) at once; each result still matches the oracle.  The launchers' one-time state is set
    up race-free, and the per-size occupancy cache is one atomic word."""
    import threading
    fmt = synth.Q4_K
    shapes = [(300, 2048), (200, 8192), (129, 4096), (77, 12288)]
    data = []
    for i, (rows, cols) in enumerate(shapes):
        blocks = synth.quant_matrix(fmt, rows, cols, seed=12, stream=900 + i)
        x = synth.normal_f32(cols, seed=12, stream=950 + i)
        ref, nrm = oracle.gemv(fmt, rows, cols, blocks, x.astype(np.float64))
        data.append((rows, cols, dev(blocks), dev(x.astype(np.float32)), ref, nrm))
    outs = [None] * len(shapes)
    errors = []

    def work(i):
        try:
            rows, cols, wb, xd, _, _ = data[i]
            st = torch.cuda.Stream()
            y = torch.empty(rows, dtype=torch.float32, device="cuda")
            for _ in range(25):
                nt.nt_gemv_q(fmt, rows, cols, wb.data_ptr(), xd.data_ptr(), y.data_ptr(), st.cuda_stream)
            st.synchronize()
            outs[i] = host(y)
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i, (rows, cols, _, _, ref, nrm) in enumerate(data):
        check_rel(outs[i], ref, nrm, what=f"thread {i} {rows}x{cols}")
