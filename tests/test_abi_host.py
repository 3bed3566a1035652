"""The C ABI library loads, exports every symbol include/nt.h declares, and rejects
bad arguments on the host before anything is enqueued (CPU only: none of these
calls reaches the GPU)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import quantized_weight_streaming_dequant_amd as nt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nt.h")


def declared_functions() -> list[str]:
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nt_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_path_calls():
    names = declared_functions()
    for need in ("nt_gemv_q", "nt_rmsnorm", "nt_rope", "nt_attn_decode", "nt_swiglu", "nt_decode_layer",
                 "nt_stream_layers", "nt_dequant"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(nt.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(nt.EXPORTS) == declared_functions()


def test_block_geometry():
    assert [nt.nt_block_elems(f) for f in range(10)] == [32, 32, 256, 256, 256, 1, 1, 256, 32, 256]
    assert [nt.nt_block_bytes(f) for f in range(10)] == [34, 18, 144, 210, 176, 2, 4, 144, 34, 176]
    assert nt.nt_matrix_bytes(nt.Q8_0T, 14336, 4096) == nt.nt_matrix_bytes(nt.Q8_0, 14336, 4096)
    assert nt.nt_matrix_bytes(nt.Q4_KT, 28672, 8192) == nt.nt_matrix_bytes(nt.Q4_K, 28672, 8192)
    assert nt.nt_matrix_bytes(nt.F16, 28672, 8192) == 2 * 28672 * 8192
    assert nt.nt_matrix_bytes(nt.Q5_K, 28672, 8192) == 161_480_704
    assert nt.nt_matrix_bytes(nt.Q6_K, 8192, 28672) == 192_675_840
    assert nt.nt_matrix_bytes(nt.Q4_K, 28672, 8192) == 132_120_576


@pytest.mark.parametrize("call,code", [
    (lambda: nt.nt_gemv_q(12, 16, 256, 16, 16, 16), nt.NT_EFORMAT),
    (lambda: nt.nt_gemv_q(nt.Q4_K, 16, 100, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemv_q(nt.Q4_K, 0, 256, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemv_q(nt.Q4_K, 16, 65536, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemv_q(nt.Q8_0, 16, 256, None, 16, 16), nt.NT_EINVAL),
    (lambda: nt.nt_gemv_q(nt.Q8_0, 16, 256, 18, 16, 16), nt.NT_EALIGN),
    (lambda: nt.nt_dequant(nt.Q6_K, 4, 255, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemv_q(11, 16, 256, 16, 16, 16), nt.NT_EFORMAT),
    (lambda: nt.nt_gemv_q(nt.Q8_0T, 16, 224, 16, 16, 16), nt.NT_ESHAPE),  # Q8_0T rows: multiples of 256 columns
    (lambda: nt.nt_repack(nt.Q8_0T, 16, 96, 16, 4096, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_repack(nt.Q4_K, 16, 256, 16, 4096, 16), nt.NT_EFORMAT),  # Q4_KT is the only target
    (lambda: nt.nt_repack(nt.Q4_KT, 16, 200, 16, 4096, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_repack(nt.Q4_KT, 0, 256, 16, 4096, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_repack(nt.Q4_KT, 16, 256, None, 4096, 16), nt.NT_EINVAL),
    (lambda: nt.nt_repack(nt.Q4_KT, 16, 256, 24, 4096, 16), nt.NT_EALIGN),
    (lambda: nt.nt_repack(nt.Q4_KT, 16, 256, 4096, 4096 + 2304 - 16, 16), nt.NT_EINVAL),  # overlap
    (lambda: nt.nt_gemv_q(nt.F16, 16, 40, 16, 16, 16), nt.NT_ESHAPE),  # F16/F32 columns: multiples of 32
    (lambda: nt.nt_gemm_q(nt.F32, 16, 48, 2, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_dequant(nt.F16, 4, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_layer_cosine(0, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_layer_cosine((1 << 24) + 1, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_layer_cosine(16, None, 16, 16), nt.NT_EINVAL),
    (lambda: nt.nt_layer_cosine(16, 16, 18, 16), nt.NT_EALIGN),
    (lambda: nt.nt_read_probe(16, 0, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_read_probe(16, 24, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_read_probe(None, 16, 16), nt.NT_EINVAL),
    (lambda: nt.nt_read_probe(8, 16, 16), nt.NT_EALIGN),
    (lambda: nt.nt_gemm_q(13, 16, 256, 2, 16, 16, 16), nt.NT_EFORMAT),
    (lambda: nt.nt_gemm_q(nt.Q4_K, 16, 256, 0, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemm_q(nt.Q4_K, 16, 256, nt.GEMM_MAX_TOK + 1, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemm_q(nt.Q4_K, 16, 200, 2, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemm_q(nt.Q4_K, 0, 256, 2, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemm_q(nt.Q8_0, 16, 256, 2, 16, None, 16), nt.NT_EINVAL),
    (lambda: nt.nt_gemm_q(nt.Q8_0, 16, 256, 2, 16, 24, 16), nt.NT_EALIGN),
    (lambda: nt.nt_rope(8, 127, 0, 5e5, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_rope(8, 128, -1, 5e5, 16), nt.NT_EINVAL),
    (lambda: nt.nt_attn_decode(64, 8, 64, 10, 16, 16, 16, 16, 16, 256, 1 << 20), nt.NT_ESHAPE),
    (lambda: nt.nt_attn_decode(64, 8, 128, 17, 16, 16, 16, 16, 16, 256, 1 << 20), nt.NT_ESHAPE),
    (lambda: nt.nt_attn_decode(64, 8, 128, 16, 16, 16, 16, 16, 16, 128, 1 << 20), nt.NT_EALIGN),
    (lambda: nt.nt_attn_decode(60, 8, 128, 16, 16, 16, 16, 16, 16, 256, 1 << 20), nt.NT_ESHAPE),
    (lambda: nt.nt_attn_decode(64, 8, 128, 16, 16, 16, 16, 16, 16, 256, 8), nt.NT_EINVAL),
    (lambda: nt.nt_attn_decode(64, 8, 128, 16, 20, 16, 16, 16, 16, 256, 1 << 20), nt.NT_ESHAPE),  # max_ctx % 8
    (lambda: nt.nt_attn_decode(64, 8, 128, 16, 2 * nt.NT_MAX_CTX, 16, 16, 16, 16, 256, 1 << 30), nt.NT_ESHAPE),
    (lambda: nt.nt_swiglu(0, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_rmsnorm(100, None, 16, 1e-5, 16), nt.NT_EINVAL),
    (lambda: nt.nt_argmax(0, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_embed_row(nt.Q4_K, 10, 100, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_stream_create(None, 256, 1024), nt.NT_EINVAL),
    (lambda: nt.nt_stream_create(256, 256, 1024), nt.NT_EINVAL),
    (lambda: nt.nt_stream_create(256, 512 + 16, 1024), nt.NT_EALIGN),
    # rows past 2^30 (row-group indices stay in 32-bit range inside the kernels)
    (lambda: nt.nt_gemv_q(nt.Q4_0, nt.NT_MAX_ROWS + 1, 32, 16, 16, 16), nt.NT_ESHAPE),
    (lambda: nt.nt_gemm_q(nt.Q4_0, nt.NT_MAX_ROWS + 1, 32, 2, 16, 16, 16), nt.NT_ESHAPE),
    # the greedy head
    (lambda: nt.nt_lm_head(14, 1000, 1024, 256, 256, 1e-5, 256, 256, 256, 256, 256), nt.NT_EFORMAT),
    (lambda: nt.nt_lm_head(nt.Q4_K, 1000, 1000, 256, 256, 1e-5, 256, 256, 256, 256, 256), nt.NT_ESHAPE),
    (lambda: nt.nt_lm_head(nt.Q4_K, 0, 1024, 256, 256, 1e-5, 256, 256, 256, 256, 256), nt.NT_ESHAPE),
    (lambda: nt.nt_lm_head(nt.Q4_K, nt.NT_MAX_ROWS + 1, 1024, 256, 256, 1e-5, 256, 256, 256, 256, 256), nt.NT_ESHAPE),
    (lambda: nt.nt_lm_head(nt.Q4_K, 1000, 1024, 256, None, 1e-5, 256, 256, 256, 256, 256), nt.NT_EINVAL),
    (lambda: nt.nt_lm_head(nt.Q4_K, 1000, 1024, 256, 256, -1.0, 256, 256, 256, 256, 256), nt.NT_EINVAL),
    (lambda: nt.nt_lm_head(nt.Q4_K, 1000, 1024, 256, 256, 1e-5, 256, 256, 256, 256, 8), nt.NT_EINVAL),
    (lambda: nt.nt_lm_head(nt.Q4_K, 1000, 1024, 264, 256, 1e-5, 256, 256, 256, 256, 256), nt.NT_EALIGN),
    (lambda: nt.nt_lm_head(nt.Q4_K, 1000, 1024, 256, 256, 1e-5, 256, 256, 256, 128, 256), nt.NT_EALIGN),
])
def test_bad_arguments_are_rejected(call, code):
    with pytest.raises(nt.NtError) as ei:
        call()
    assert ei.value.code == code
    assert nt.last_error()


def _shape(**kw):
    base = dict(dim=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn_dim=14336, max_ctx=1024, eps=1e-5,
                rope_theta=5e5)
    base.update(kw)
    return nt.LayerShape(*[base[k] for k in ("dim", "n_q_heads", "n_kv_heads", "head_dim", "ffn_dim", "max_ctx",
                                              "eps", "rope_theta")])


def _weights(fmt=nt.Q8_0, ptr=4096):
    w = nt.LayerWeights()
    for i in range(nt.W_COUNT):
        w.fmt[i] = fmt
        w.w[i] = ptr
    w.attn_norm = ptr
    w.ffn_norm = ptr
    return w


@pytest.mark.parametrize("shape_kw,wfix,pos,code", [
    (dict(head_dim=64), None, 0, nt.NT_ESHAPE),
    (dict(n_q_heads=30), None, 0, nt.NT_ESHAPE),
    (dict(n_q_heads=96, n_kv_heads=8), None, 0, nt.NT_ESHAPE),  # group of 12
    (dict(dim=4000), None, 0, nt.NT_ESHAPE),
    (dict(ffn_dim=40960), None, 0, nt.NT_ESHAPE),
    ({}, None, 1024, nt.NT_ESHAPE),
    (dict(max_ctx=1020), None, 0, nt.NT_ESHAPE),
    (dict(max_ctx=2 * nt.NT_MAX_CTX), None, 0, nt.NT_ESHAPE),
    ({}, None, -1, nt.NT_ESHAPE),
    ({}, "badfmt", 0, nt.NT_EFORMAT),
    ({}, "mixed_ffn", 0, nt.NT_EFORMAT),
    ({}, "misaligned", 0, nt.NT_EALIGN),
    ({}, "null", 0, nt.NT_EINVAL),
])
def test_decode_layer_checks(shape_kw, wfix, pos, code):
    shp = _shape(**shape_kw)
    w = _weights()
    if wfix == "badfmt":
        w.fmt[3] = 11
    elif wfix == "mixed_ffn":
        w.fmt[nt.W_GATE] = nt.Q4_K
    elif wfix == "misaligned":
        w.w[2] = 4096 + 8
    elif wfix == "null":
        w.w[5] = None
    with pytest.raises(nt.NtError) as ei:
        nt.nt_decode_layer(w, shp, pos, 4096, 4096, 4096, 4096, 1 << 30)
    assert ei.value.code == code


@pytest.mark.parametrize("shape_kw,wfix,code", [
    (dict(head_dim=64), None, nt.NT_ESHAPE),
    (dict(ffn_dim=40960), None, nt.NT_ESHAPE),
    ({}, "mixed_ffn", nt.NT_EFORMAT),
    ({}, "null_h", nt.NT_EINVAL),
    ({}, "misaligned_h", nt.NT_EALIGN),
])
def test_ffn_up_checks(shape_kw, wfix, code):
    shp = _shape(**shape_kw)
    w = _weights()
    h = 4096
    if wfix == "mixed_ffn":
        w.fmt[nt.W_GATE] = nt.Q4_K
    elif wfix == "null_h":
        h = None
    elif wfix == "misaligned_h":
        h = 4096 + 4
    with pytest.raises(nt.NtError) as ei:
        nt.nt_ffn_up(w, shp, h, 4096)
    assert ei.value.code == code


def test_layer_k_checks():
    shp = _shape()
    w = _weights()
    for pos, k, code in ((0, 0, nt.NT_ESHAPE), (0, nt.GEMM_MAX_TOK + 1, nt.NT_ESHAPE), (1020, 5, nt.NT_ESHAPE),
                         (-1, 2, nt.NT_ESHAPE)):
        with pytest.raises(nt.NtError) as ei:
            nt.nt_decode_layer_k(w, shp, pos, k, 4096, 4096, 4096, 4096, 1 << 30)
        assert ei.value.code == code, (pos, k)
    with pytest.raises(nt.NtError) as ei:
        nt.nt_decode_layer_k(w, shp, 0, 4, 4096, 4096, 4096, 4096, 1024)
    assert ei.value.code == nt.NT_EINVAL  # workspace too small
    assert nt.nt_decode_layer_k_ws_bytes(shp, 0) == 0 and nt.nt_decode_layer_k_ws_bytes(shp, 9) == 0
    # the k-token workspace holds k rows of every stage and k tokens' attention partials
    assert nt.nt_decode_layer_k_ws_bytes(shp, 8) > 8 * 4 * (4096 + 14336)
    off = nt.nt_decode_layer_k_ws_offsets(shp, 4)
    assert all(v % 256 == 0 for v in off.values())


def test_workspace_sizes_and_offsets():
    shp = _shape()
    ws = nt.nt_decode_layer_ws_bytes(shp)
    off = nt.nt_decode_layer_ws_offsets(shp)
    assert all(v % 256 == 0 for v in off.values())
    assert off["q"] < off["o"] < off["h1"] < off["a"] < off["part"] < ws
    assert ws >= 4 * (2 * 4096 + 4096 + 14336)
    assert nt.nt_attn_decode_ws_bytes(64, 8, 128, 4224) > 4 * 64 * 130
    assert nt.nt_decode_token_ws_bytes(shp) >= ws


def test_layer_workspace_too_small():
    with pytest.raises(nt.NtError) as ei:
        nt.nt_decode_layer(_weights(), _shape(), 5, 4096, 4096, 4096, 4096, 1024)
    assert ei.value.code == nt.NT_EINVAL


def test_header_constants_match_binding():
    import re
    text = open(HEADER).read()
    for name in ("NT_MAX_CTX", "NT_GEMV_MAX_COLS", "NT_LM_HEAD_WS_BYTES"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(nt, name), name
    m = re.search(r"#define\s+NT_MAX_ROWS\s+\(1 << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == nt.NT_MAX_ROWS


def test_stream_threshold_policy_round_trips():
    """The GEMV launch policy's streamed-path threshold: default 10^8 weights, returned as the
    previous value on every set, left alone by a negative argument (host state only)."""
    prev = nt.nt_set_stream_min_weights(-1)
    assert prev == 10 ** 8
    try:
        assert nt.nt_set_stream_min_weights(0) == 10 ** 8
        assert nt.nt_set_stream_min_weights(-5) == 0
        assert nt.nt_set_stream_min_weights(12345) == 0
        assert nt.nt_set_stream_min_weights(-1) == 12345
    finally:
        nt.nt_set_stream_min_weights(prev)
