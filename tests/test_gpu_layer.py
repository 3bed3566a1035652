"""GPU parity of the fused decode layer, the greedy token step and layer streaming
(MI355X only), through the C ABI.

Stage-wise, teacher-forced acceptance (each stage judged on the GPU's own input
to it): the fp16 K/V written at slot pos within the GEMV tolerance of the exact
value plus half a binary16 step; the rotated query, attention output, h1,
SwiGLU output and h2 each within 1e-3 of their normalisers.  Streaming must be bit-identical to
running the same layers resident.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
import quantized_weight_streaming_dequant_amd as nt
import synth
from quantized_weight_streaming_dequant_amd import torch_glue as tg
from synth import recipes
from tests.gpu_util import (check_layer_stages, check_rel, dev, host, same_value, say, stream, v_from_device,
                            v_to_device)

pytestmark = pytest.mark.gpu


class DeviceLayer:
    """One layer's tensors on the device, generated from the seed streams."""

    def __init__(self, shape, mix, layer, n_slots, seed=0):
        self.shape, self.mix, self.layer = shape, mix, layer
        self.host = recipes.layer_arrays(shape, mix, layer, seed)
        self.dev = {k: dev(v) for k, v in self.host.items()}
        self.kc_host = recipes.kv_cache_array(shape, layer, "k", n_slots, seed)
        self.vc_host = recipes.kv_cache_array(shape, layer, "v", n_slots, seed)
        self.kc = dev(self.kc_host)
        self.vc = dev(v_to_device(self.vc_host, shape.n_kv_heads, shape.max_ctx))

    def weights(self):
        return tg.layer_weights([self.mix[n] for n in recipes.TENSORS], [self.dev[n] for n in recipes.TENSORS],
                                self.dev["attn_norm"], self.dev["ffn_norm"])


def run_layer_and_check(shape, mix, pos, n_slots, layer=0, sample_rows=None):
    say(f"decode layer dim={shape.dim} nq={shape.n_q_heads} nkv={shape.n_kv_heads} ffn={shape.ffn_dim} pos={pos}")
    L = DeviceLayer(shape, mix, layer, n_slots)
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    off = nt.nt_decode_layer_ws_offsets(shp)
    h0 = recipes.hidden_input(shape.dim)
    h = dev(h0)
    nt.nt_decode_layer(L.weights(), shp, pos, h.data_ptr(), L.kc.data_ptr(), L.vc.data_ptr(), ws.data_ptr(), wsb,
                       stream())
    torch.cuda.synchronize()
    nq = shape.n_q_heads * shape.head_dim

    def wsf(name, n):
        return ws[off[name]:off[name] + 4 * n].view(torch.float32).cpu().numpy()

    g_q, g_o, g_h1, g_a = wsf("q", nq), wsf("o", nq), wsf("h1", shape.dim), wsf("a", shape.ffn_dim)
    g_h2 = host(h)
    kc, vc = host(L.kc), v_from_device(host(L.vc), shape.n_kv_heads, shape.max_ctx)
    g_k16, g_v16 = kc[:, pos, :].ravel(), vc[:, pos, :].ravel()
    # untouched cache slots stay as they were
    keep = np.ones(shape.max_ctx, bool)
    keep[pos] = False
    assert same_value(kc[:, keep], L.kc_host[:, keep]) and same_value(vc[:, keep], L.vc_host[:, keep])

    st = oracle.decode_layer(L.host, mix, shape, pos, h0, L.kc_host, L.vc_host,
                             forced={"k16": g_k16, "v16": g_v16, "q": g_q, "o": g_o, "h1": g_h1, "a": g_a})
    res = check_layer_stages(st, {"k16": g_k16, "v16": g_v16, "q": g_q, "o": g_o, "h1": g_h1, "a": g_a,
                                  "h2": g_h2})
    # free-running (no forcing) end-to-end error, reported only
    free = oracle.decode_layer(L.host, mix, shape, pos, h0, L.kc_host, L.vc_host)
    rel = np.max(np.abs(g_h2 - free["h2"]) / (free["h2_nrm"]))
    say("  stage worst rel errors " + ", ".join(f"{k} {v:.1e}" for k, v in res.items()) + f"; free-running h2 {rel:.1e}")
    return res


def test_layer_8b_q8_0_full_size():
    """Llama-3-8B-shaped layer, Q8_0, pos 1023 over a 1024-slot fp16 cache."""
    run_layer_and_check(recipes.LLAMA3_8B, recipes.MIX_Q8_0, pos=1023, n_slots=1024)


def test_layer_70b_q4_k_m_full_size():
    """Llama-3.1-70B-shaped layer in the Q4_K_M mix at pos 4096 over a 4096-slot prefill."""
    run_layer_and_check(recipes.LLAMA31_70B, recipes.MIX_Q4_K_M, pos=4096, n_slots=4096)


def test_layer_70b_q6_k_full_size():
    run_layer_and_check(recipes.LLAMA31_70B, recipes.MIX_Q6_K, pos=4200, n_slots=4096, layer=3)


def test_layer_8b_f16_full_size():
    """The Llama-3-8B-shaped layer with unquantized F16 weights (436 MB)."""
    run_layer_and_check(recipes.LLAMA3_8B, recipes.MIX_F16, pos=1000, n_slots=1000)


def test_layer_70b_q5_k_m_full_size():
    """The 70B-shaped layer in the Q5_K_M mix (Q5_K, with Q6_K for attn_v and ffn_down)."""
    run_layer_and_check(recipes.LLAMA31_70B, recipes.MIX_Q5_K_M, pos=4100, n_slots=4096, layer=5)


SMALL = recipes.LayerShape(dim=1024, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn_dim=2816, max_ctx=96)


@pytest.mark.parametrize("mix,pos", [(recipes.MIX_Q4_K_M, 0), (recipes.MIX_Q8_0, 50), (recipes.MIX_Q6_K, 95),
                                     ({n: synth.Q4_0 for n in recipes.TENSORS}, 17), (recipes.MIX_Q5_K_M, 33),
                                     ({n: synth.Q5_K for n in recipes.TENSORS}, 64), (recipes.MIX_F16, 40),
                                     (recipes.MIX_F32, 71),
                                     # F16 attention projections over a Q4_K_M FFN, Q8_0 q/k with an F32 v
                                     ({**recipes.MIX_Q4_K_M, "q": synth.F16, "k": synth.F16, "v": synth.F16,
                                       "o": synth.F16}, 12),
                                     ({**recipes.MIX_Q8_0, "v": synth.F32}, 90)])
def test_layer_small_shapes(mix, pos):
    run_layer_and_check(SMALL, mix, pos=pos, n_slots=96)


# Every launch that the streamed path can take, forced onto it (the launch policy otherwise keeps
# launches under 10^8 weights on the register path): its q/k/v + RoPE, gate/up + SwiGLU and
# residual epilogues, the x and gain slices staged through its rings, partial column slices
# (dim 1024 against 4096- or 2048-column slices) and full ones (the 8B shape).
@pytest.mark.parametrize("shape,mix,pos", [(SMALL, recipes.MIX_Q8_0, 50), (SMALL, recipes.MIX_Q6_K, 95),
                                           (SMALL, {n: synth.Q4_0 for n in recipes.TENSORS}, 17),
                                           (SMALL, recipes.MIX_Q4_K_M, 3), (recipes.LLAMA3_8B, recipes.MIX_Q8_0, 700)])
def test_layer_streamed_path_forced(shape, mix, pos):
    prev = nt.nt_set_stream_min_weights(0)
    try:
        run_layer_and_check(shape, mix, pos=pos, n_slots=min(shape.max_ctx, 1000))
    finally:
        nt.nt_set_stream_min_weights(prev)


@pytest.mark.parametrize("shape,mix", [(SMALL, recipes.MIX_Q4_K_M), (recipes.LLAMA31_70B, recipes.MIX_Q4_K_M),
                                       (recipes.LLAMA3_8B, recipes.MIX_Q8_0)])
def test_ffn_up_entry_matches_layer(shape, mix):
    """nt_ffn_up on the layer's own h1 reproduces the SwiGLU output nt_decode_layer leaves in
    its workspace, bit for bit (the same launch)."""
    say(f"ffn_up entry dim={shape.dim} ffn={shape.ffn_dim}")
    L = DeviceLayer(shape, mix, 0, 8)
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    off = nt.nt_decode_layer_ws_offsets(shp)
    h = dev(recipes.hidden_input(shape.dim))
    nt.nt_decode_layer(L.weights(), shp, 7, h.data_ptr(), L.kc.data_ptr(), L.vc.data_ptr(), ws.data_ptr(), wsb, stream())
    h1 = ws[off["h1"]:off["h1"] + 4 * shape.dim].view(torch.float32).clone()
    a_layer = host(ws[off["a"]:off["a"] + 4 * shape.ffn_dim].view(torch.float32))
    a = torch.full((shape.ffn_dim,), float("nan"), dtype=torch.float32, device="cuda")
    nt.nt_ffn_up(L.weights(), shp, h1.data_ptr(), a.data_ptr(), stream())
    assert same_value(host(a), a_layer)


# ------------------------------------------------------------------ model, token, streaming

class Model:
    """A small model in one contiguous blob per layer; some layers in pinned host memory."""

    def __init__(self, shape, mix, n_layers, vocab, streamed=(), n_slots=None, seed=0):
        self.shape, self.mix, self.n_layers, self.vocab = shape, mix, n_layers, vocab
        self.lay = recipes.blob_layout(shape, mix)
        self.blobs_dev = []
        self.blobs_host = []
        for l in range(n_layers):
            hb = torch.empty(self.lay.nbytes, dtype=torch.uint8, pin_memory=True)
            recipes.fill_layer_blob(hb.data_ptr(), shape, mix, l, seed, self.lay)
            self.blobs_host.append(hb)
            self.blobs_dev.append(hb.cuda())
        self.streamed = set(streamed)
        n_slots = n_slots if n_slots is not None else shape.max_ctx
        self.kc0 = [recipes.kv_cache_array(shape, l, "k", n_slots, seed) for l in range(n_layers)]
        self.vc0 = [recipes.kv_cache_array(shape, l, "v", n_slots, seed) for l in range(n_layers)]
        self.embd = synth.quant_matrix(synth.Q4_K, vocab, shape.dim, seed, recipes.stream_id(recipes.GLOBAL_LAYER, 0))
        self.out = synth.quant_matrix(synth.Q4_K, vocab, shape.dim, seed, recipes.stream_id(recipes.GLOBAL_LAYER, 1))
        self.onorm = synth.uniform_f32(shape.dim, seed, recipes.stream_id(recipes.GLOBAL_LAYER, 2), 0.9, 1.1)
        self.embd_d, self.out_d, self.onorm_d = dev(self.embd), dev(self.out), dev(self.onorm)

    def caches(self):
        return ([dev(k) for k in self.kc0],
                [dev(v_to_device(v, self.shape.n_kv_heads, self.shape.max_ctx)) for v in self.vc0])

    def plan(self, kcs, vcs, streamed=None, skip=(), layers=None, files=None):
        """layers: the layer indices the plan lists (default all), in order; files: layer ->
        (fd, offset) for layers read from a file."""
        files = files or {}
        streamed = self.streamed if streamed is None else streamed
        layers = range(self.n_layers) if layers is None else layers
        shp = tg.layer_shape(self.shape)
        lay = tg.layer_layout(self.lay.offset_list(), self.lay.fmt_list(), self.lay.nbytes)
        ents = []
        for l in layers:
            if l in files:
                ents.append((0, nt.TIER_FILE, kcs[l].data_ptr(), vcs[l].data_ptr(), files[l][0], files[l][1]))
            elif l in streamed:
                ents.append((self.blobs_host[l].data_ptr(), False, kcs[l].data_ptr(), vcs[l].data_ptr()))
            else:
                ents.append((self.blobs_dev[l].data_ptr(), True, kcs[l].data_ptr(), vcs[l].data_ptr()))
        return tg.model_plan(shp, lay, ents, skip={i for i, l in enumerate(layers) if l in skip})

    def head(self):
        return nt.ModelHead(synth.Q4_K, self.embd_d.data_ptr(), self.vocab, self.onorm_d.data_ptr(), synth.Q4_K,
                            self.out_d.data_ptr())


def decode_tokens(model, streamed, tok0, pos0, n_tokens, staging=None, skip=(), layers=None, files=None, bounce=None):
    kcs, vcs = model.caches()
    plan, keep = model.plan(kcs, vcs, streamed, skip, layers, files)
    shp = tg.layer_shape(model.shape)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(model.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(model.vocab, dtype=torch.float32, device="cuda")
    tok = torch.tensor([tok0], dtype=torch.int32, device="cuda")
    compute = torch.cuda.Stream()
    copy = torch.cuda.Stream()
    st = None
    if streamed or files:
        st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), staging[0].numel())
    if files:
        nt.nt_stream_set_bounce(st, bounce[0].data_ptr(), bounce[1].data_ptr(), bounce[0].numel(), 3)
    toks, hs, lgs = [], [], []
    stats = nt.StreamStats()
    try:
        for i in range(n_tokens):
            torch.cuda.synchronize()
            nt.nt_decode_token(st, plan, model.head(), pos0 + i, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                               ws.data_ptr(), wsb, compute.cuda_stream, copy.cuda_stream, stats)
            torch.cuda.synchronize()
            toks.append(int(tok.cpu()[0]))
            hs.append(h.cpu().numpy().copy())
            lgs.append(logits.cpu().numpy().copy())
    finally:
        if st is not None:
            torch.cuda.synchronize()
            nt.nt_stream_destroy(st)
    return toks, hs, lgs, [host(k) for k in kcs], [host(v) for v in vcs], stats


TINY = recipes.LayerShape(dim=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn_dim=2048, max_ctx=64)


def test_token_step_and_streaming_bit_identical():
    say("token step: resident vs streamed (layers 1 and 3 of 4)")
    m = Model(TINY, recipes.MIX_Q4_K_M, 4, vocab=1000, n_slots=32)
    tok0 = synth.uniform_index(1000, 0, 77)
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    a = decode_tokens(m, set(), tok0, 32, 3)
    b = decode_tokens(m, {1, 3}, tok0, 32, 3, staging)
    assert a[0] == b[0]
    for x, y in zip(a[1], b[1]):
        assert same_value(x, y)
    for x, y in zip(a[2], b[2]):
        assert same_value(x, y)
    for x, y in zip(a[3] + a[4], b[3] + b[4]):
        assert same_value(x, y)
    assert b[5].layers_streamed == 2
    say(f"  tokens {a[0]}")
    # the checker: logits of the last token from the GPU's final hidden state, and the greedy pick
    h_last = a[1][-1]
    n = oracle.rmsnorm(h_last, m.onorm, TINY.eps)
    ref, nrm = oracle.gemv(synth.Q4_K, 1000, TINY.dim, m.out, n)
    check_rel(a[2][-1], ref, nrm, what="logits")
    best = ref.max()
    assert ref[a[0][-1]] >= best - 1e-3 * nrm[a[0][-1]]


def test_token_step_matches_layer_calls():
    """nt_decode_token = embedding row, then the layers, then the head, with the same kernels."""
    say("token step vs per-layer calls")
    m = Model(TINY, recipes.MIX_Q4_K_M, 3, vocab=500, n_slots=20)
    tok0 = 123
    toks, hs, lgs, kcs, vcs, _ = decode_tokens(m, set(), tok0, 20, 1)
    # replay by hand through nt_embed_row + nt_decode_layer
    kd, vd = m.caches()
    shp = tg.layer_shape(TINY)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(TINY.dim, dtype=torch.float32, device="cuda")
    t = torch.tensor([tok0], dtype=torch.int32, device="cuda")
    nt.nt_embed_row(synth.Q4_K, 500, TINY.dim, m.embd_d.data_ptr(), t.data_ptr(), h.data_ptr(), stream())
    assert same_value(host(h), oracle.dequant_f32(synth.Q4_K, 500, TINY.dim, m.embd)[tok0])
    for l in range(3):
        blob = m.blobs_dev[l]
        mats = [blob[m.lay.offsets[n]:] for n in recipes.TENSORS]
        w = tg.layer_weights(m.lay.fmt_list(), mats, blob[m.lay.offsets["attn_norm"]:].view(torch.float32),
                             blob[m.lay.offsets["ffn_norm"]:].view(torch.float32))
        nt.nt_decode_layer(w, shp, 20, h.data_ptr(), kd[l].data_ptr(), vd[l].data_ptr(), ws.data_ptr(), wsb, stream())
    assert same_value(host(h), hs[0])
    for l in range(3):
        assert same_value(host(kd[l]), kcs[l]) and same_value(host(vd[l]), vcs[l])


def decode_tokens_async(model, streamed, tok0, pos0, n_tokens, staging, sleep_compute=0, sleep_copy=0):
    """n_tokens greedy tokens enqueued back to back with no host synchronisation between them;
    each token's outputs are copied on the compute stream into per-token buffers.  Optional
    bounded spin kernels (torch.cuda._sleep, in GPU clock cycles) at the start of each call on
    the compute or the copy stream make that stream lag the other by about a millisecond."""
    kcs, vcs = model.caches()
    plan, keep = model.plan(kcs, vcs, streamed)
    shp = tg.layer_shape(model.shape)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(model.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(model.vocab, dtype=torch.float32, device="cuda")
    tok = torch.tensor([tok0], dtype=torch.int32, device="cuda")
    H = torch.zeros(n_tokens, model.shape.dim, dtype=torch.float32, device="cuda")
    LG = torch.zeros(n_tokens, model.vocab, dtype=torch.float32, device="cuda")
    T = torch.zeros(n_tokens, dtype=torch.int32, device="cuda")
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), staging[0].numel()) if streamed else None
    stats = nt.StreamStats()
    torch.cuda.synchronize()
    try:
        for i in range(n_tokens):
            if sleep_compute:
                with torch.cuda.stream(compute):
                    torch.cuda._sleep(sleep_compute)
            if sleep_copy:
                with torch.cuda.stream(copy):
                    torch.cuda._sleep(sleep_copy)
            nt.nt_decode_token(st, plan, model.head(), pos0 + i, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                               ws.data_ptr(), wsb, compute.cuda_stream, copy.cuda_stream, stats)
            with torch.cuda.stream(compute):
                H[i].copy_(h)
                LG[i].copy_(logits)
                T[i:i + 1].copy_(tok)
        torch.cuda.synchronize()
    finally:
        if st is not None:
            torch.cuda.synchronize()
            nt.nt_stream_destroy(st)
    return host(T).tolist(), host(H), host(LG), [host(k) for k in kcs], [host(v) for v in vcs]


@pytest.mark.parametrize("sleep_compute,sleep_copy", [(0, 0), (4_000_000, 0), (0, 4_000_000)])
def test_streaming_staging_reuse_under_delays(sleep_compute, sleep_copy):
    """Five distinct streamed layers through two staging buffers (so each buffer holds a different
    layer on every reuse), four tokens enqueued back to back without a host synchronisation, with
    the compute stream held back (copies run ahead: only the buffers' free events keep them from
    overwriting a layer before it ran) or the copy stream held back (only the ready events keep
    compute from running a layer on the previous occupant's weights): bit for bit the resident run."""
    say(f"staging reuse: 5 streamed layers, sleeps compute {sleep_compute} copy {sleep_copy} cycles")
    m = Model(TINY, recipes.MIX_Q4_K_M, 6, vocab=1000, n_slots=24)
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    tok0 = synth.uniform_index(1000, 0, 83)
    a = decode_tokens_async(m, set(), tok0, 24, 4, staging)
    b = decode_tokens_async(m, {1, 2, 3, 4, 5}, tok0, 24, 4, staging, sleep_compute, sleep_copy)
    assert a[0] == b[0]
    assert same_value(a[1], b[1]) and same_value(a[2], b[2])
    for x, y in zip(a[3] + a[4], b[3] + b[4]):
        assert same_value(x, y)


def test_stream_prefetch_from_changed_entries_is_not_used():
    """The streamer prefetches the first streamed layers of the next token at the end of a call;
    if the caller then points those entries at other blobs (same plan array, same streamed list),
    the prefetched copies are dropped and the new blobs are used."""
    say("streamer: changed plan entries after a prefetch")
    m = Model(TINY, recipes.MIX_Q4_K_M, 4, vocab=1000, n_slots=24)
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    kcs, vcs = m.caches()
    plan, keep = m.plan(kcs, vcs, {1, 3})
    shp = tg.layer_shape(TINY)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(TINY.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(1000, dtype=torch.float32, device="cuda")
    tok = torch.tensor([7], dtype=torch.int32, device="cuda")
    cs, cp = torch.cuda.Stream(), torch.cuda.Stream()
    st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), m.lay.nbytes)
    try:
        nt.nt_decode_token(st, plan, m.head(), 24, tok.data_ptr(), logits.data_ptr(), h.data_ptr(), ws.data_ptr(),
                           wsb, cs.cuda_stream, cp.cuda_stream)
        torch.cuda.synchronize()
        # swap the two streamed entries' blobs in place: layer 1 now runs layer 3's weights and back
        b1, b3 = keep[1].blob, keep[3].blob
        keep[1].blob, keep[3].blob = b3, b1
        tok.fill_(11)
        nt.nt_decode_token(st, plan, m.head(), 25, tok.data_ptr(), logits.data_ptr(), h.data_ptr(), ws.data_ptr(),
                           wsb, cs.cuda_stream, cp.cuda_stream)
        torch.cuda.synchronize()
        got_h = host(h).copy()
    finally:
        torch.cuda.synchronize()
        nt.nt_stream_destroy(st)
    # the same two tokens with fresh caches, resident, the second with layers 1 and 3 swapped the same way
    shp_layers = []
    for l in range(4):
        blob = m.blobs_dev[{1: 3, 3: 1}.get(l, l)]
        mats = [blob[m.lay.offsets[n]:] for n in recipes.TENSORS]
        shp_layers.append(tg.layer_weights(m.lay.fmt_list(), mats, blob[m.lay.offsets["attn_norm"]:].view(torch.float32),
                                           blob[m.lay.offsets["ffn_norm"]:].view(torch.float32)))
    kd2, vd2 = m.caches()
    plan2, keep2 = m.plan(kd2, vd2, set())
    t2 = torch.tensor([7], dtype=torch.int32, device="cuda")
    h2 = torch.zeros(TINY.dim, dtype=torch.float32, device="cuda")
    nt.nt_decode_token(None, plan2, m.head(), 24, t2.data_ptr(), logits.data_ptr(), h2.data_ptr(), ws.data_ptr(), wsb,
                       stream(), stream())
    t2.fill_(11)
    nt.nt_embed_row(synth.Q4_K, 1000, TINY.dim, m.embd_d.data_ptr(), t2.data_ptr(), h2.data_ptr(), stream())
    lws = torch.zeros(nt.nt_decode_layer_ws_bytes(shp), dtype=torch.uint8, device="cuda")
    for l in range(4):
        nt.nt_decode_layer(shp_layers[l], shp, 25, h2.data_ptr(), kd2[l].data_ptr(), vd2[l].data_ptr(), lws.data_ptr(),
                           lws.numel(), stream())
    assert same_value(host(h2), got_h)


def test_layer_skip_equals_leaving_the_layers_out():
    """Skipped layers are not run: decoding with layers 1 and 2 of 4 skipped gives bit for bit
    what a plan listing only layers 0 and 3 gives, the skipped layers' caches are untouched,
    and a skipped streamed layer is not copied (layers 2 and 3 streamed, 2 skipped)."""
    say("layer skip vs a plan without the layers")
    m = Model(TINY, recipes.MIX_Q4_K_M, 4, vocab=1000, n_slots=32)
    tok0 = synth.uniform_index(1000, 0, 78)
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    a = decode_tokens(m, set(), tok0, 32, 3, skip={1, 2})
    b = decode_tokens(m, set(), tok0, 32, 3, layers=[0, 3])
    c = decode_tokens(m, {2, 3}, tok0, 32, 3, staging, skip={1, 2})
    assert a[0] == b[0] == c[0]
    for x, y, z in zip(a[1] + a[2], b[1] + b[2], c[1] + c[2]):
        assert same_value(x, y) and same_value(x, z)
    kc0 = [dev(k) for k in m.kc0]
    for l in (1, 2):
        assert same_value(a[3][l], host(kc0[l])) and same_value(c[3][l], host(kc0[l]))
    assert same_value(a[3][3], c[3][3]) and not same_value(a[3][3], host(kc0[3]))
    assert c[5].layers_streamed == 1
    # the run is still the model's: the last token's logits against the checker on the GPU's h
    n = oracle.rmsnorm(a[1][-1], m.onorm, TINY.eps)
    ref, nrm = oracle.gemv(synth.Q4_K, 1000, TINY.dim, m.out, n)
    check_rel(a[2][-1], ref, nrm, what="logits with layers skipped")


def _pinned_page_aligned(nbytes):
    """A page-locked host tensor of at least nbytes whose data starts on a 4096-byte boundary."""
    t = torch.empty(nbytes + 4096, dtype=torch.uint8, pin_memory=True)
    off = (-t.data_ptr()) % 4096
    return t[off:off + nbytes]


def test_file_tier_bit_identical(tmp_path):
    """Layers read from a file through page-locked bounce buffers (layers 1 and 3), next to a
    pinned one (2) and a resident one (0), decode bit for bit as the all-resident model."""
    import os
    say("file tier: layers 1 and 3 from a file")
    m = Model(TINY, recipes.MIX_Q4_K_M, 4, vocab=1000, n_slots=32)
    stride = (m.lay.nbytes + 4095) // 4096 * 4096
    path = tmp_path / "layers.bin"
    with open(path, "wb") as f:
        for l in (3, 1):  # file order unlike layer order
            f.write(m.blobs_host[l].numpy().tobytes())
            f.write(b"\0" * (stride - m.lay.nbytes))
    fd = os.open(path, os.O_RDONLY)
    try:
        files = {3: (fd, 0), 1: (fd, stride)}
        staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
        bounce = [_pinned_page_aligned(m.lay.nbytes) for _ in range(2)]
        tok0 = synth.uniform_index(1000, 0, 79)
        a = decode_tokens(m, set(), tok0, 32, 3)
        b = decode_tokens(m, {2}, tok0, 32, 3, staging, files=files, bounce=bounce)
        assert a[0] == b[0]
        for x, y in zip(a[1] + a[2] + a[3] + a[4], b[1] + b[2] + b[3] + b[4]):
            assert same_value(x, y)
        assert b[5].layers_streamed == 3 and b[5].h2d_bytes >= 3 * m.lay.nbytes
        # a blob past the end of the file is a host-side error, reported before its copy
        bad = {3: (fd, 0), 1: (fd, 4 * stride)}
        with pytest.raises(nt.NtError) as ei:
            decode_tokens(m, set(), tok0, 32, 1, staging, files=bad, bounce=bounce)
        assert ei.value.code == nt.NT_EHOSTMEM
    finally:
        os.close(fd)


def test_layer_cosine_calibration():
    """The calibration pass: cos(h before, h after) per layer, on the GPU, matches the checker's
    cosine of the same vectors; the kernel also meets the closed forms."""
    say("layer cosine calibration")
    for n, kind in ((1, "same"), (7, "neg"), (8192, "rand"), (28672, "rand"), (1 << 20, "rand"), (8192, "zero"),
                    (8192, "orth")):
        a = synth.normal_f32(n, 1, 7)
        b = {"same": a, "neg": -a, "rand": synth.normal_f32(n, 1, 8), "zero": np.zeros(n, np.float32)}.get(kind)
        if kind == "orth":
            r = synth.normal_f32(n, 1, 9).astype(np.float64)
            b = (r - a * (r @ a) / (a @ a.astype(np.float64))).astype(np.float32)
        out = torch.zeros(1, dtype=torch.float32, device="cuda")
        ad, bd = dev(a), dev(b)  # both alive across the call
        nt.nt_layer_cosine(n, ad.data_ptr(), bd.data_ptr(), out.data_ptr(), stream())
        got, ref = float(host(out)[0]), oracle.cosine(a, b)
        assert abs(got - ref) <= 1e-6, (n, kind, got, ref)
    m = Model(TINY, recipes.MIX_Q4_K_M, 3, vocab=100, n_slots=16)
    kd, vd = m.caches()
    shp = tg.layer_shape(TINY)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = dev(recipes.hidden_input(TINY.dim))
    cos = torch.zeros(3, dtype=torch.float32, device="cuda")
    for l in range(3):
        blob = m.blobs_dev[l]
        mats = [blob[m.lay.offsets[nm]:] for nm in recipes.TENSORS]
        w = tg.layer_weights(m.lay.fmt_list(), mats, blob[m.lay.offsets["attn_norm"]:].view(torch.float32),
                             blob[m.lay.offsets["ffn_norm"]:].view(torch.float32))
        h_in = h.clone()
        nt.nt_decode_layer(w, shp, 16, h.data_ptr(), kd[l].data_ptr(), vd[l].data_ptr(), ws.data_ptr(), wsb, stream())
        nt.nt_layer_cosine(TINY.dim, h_in.data_ptr(), h.data_ptr(), cos[l:].data_ptr(), stream())
        torch.cuda.synchronize()
        assert abs(float(host(cos)[l]) - oracle.cosine(host(h_in), host(h))) <= 1e-6


def test_streaming_70b_q6_k_layer_bit_identical():
    """A real-size Q6_K 70B layer (701.9 MB) run from pinned host memory through a staging
    buffer gives bit-identical results to the same blob run resident."""
    say("streaming a 70B Q6_K layer")
    shape = recipes.LLAMA31_70B
    m = Model(shape, recipes.MIX_Q6_K, 2, vocab=256, n_slots=4096)
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    a = decode_tokens(m, set(), 7, 4096, 2)
    b = decode_tokens(m, {1}, 7, 4096, 2, staging)
    assert a[0] == b[0]
    for x, y in zip(a[1] + a[2], b[1] + b[2]):
        assert same_value(x, y)
    assert b[5].h2d_bytes >= m.lay.nbytes


def test_stream_rejects_pageable_host_memory():
    m = Model(TINY, recipes.MIX_Q4_K_M, 2, vocab=100, n_slots=8)
    kcs, vcs = m.caches()
    pageable = np.zeros(m.lay.nbytes + 256, np.uint8)
    addr = (pageable.ctypes.data + 255) // 256 * 256
    shp = tg.layer_shape(TINY)
    lay = tg.layer_layout(m.lay.offset_list(), m.lay.fmt_list(), m.lay.nbytes)
    plan, keep = tg.model_plan(shp, lay, [(m.blobs_dev[0].data_ptr(), True, kcs[0].data_ptr(), vcs[0].data_ptr()),
                                          (addr, False, kcs[1].data_ptr(), vcs[1].data_ptr())])
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), m.lay.nbytes)
    ws = torch.zeros(nt.nt_decode_layer_ws_bytes(shp), dtype=torch.uint8, device="cuda")
    h = torch.zeros(TINY.dim, dtype=torch.float32, device="cuda")
    c1, c2 = torch.cuda.Stream(), torch.cuda.Stream()
    try:
        with pytest.raises(nt.NtError) as ei:
            nt.nt_stream_layers(st, plan, 8, h.data_ptr(), ws.data_ptr(), ws.numel(), c1.cuda_stream, c2.cuda_stream)
        assert ei.value.code == nt.NT_EHOSTMEM
    finally:
        nt.nt_stream_destroy(st)
