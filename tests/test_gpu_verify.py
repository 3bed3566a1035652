"""GPU parity of the verification pass of self-speculative decoding (MI355X only), through the
C ABI: the ntransformer overview (de.news.hada.io, "Hauptfunktionen") drafts tokens with the
VRAM-resident layers and checks them with the whole model in one pass.

* nt_decode_layer_k (k tokens at positions pos .. pos + k - 1) against k sequential
  teacher-forced checker layers: token t's checker run starts from the GPU's input row t and a
  cache holding the GPU's fp16 k/v of tokens 0 .. t - 1, and every stage is judged as in the
  single-token layer tests.
* nt_verify_tokens over a whole model: logits against the checker on the GPU's final hidden
  states, and the greedy picks equal to sequential greedy decoding.
* A self-speculative loop: draft with the resident layers (the streamed ones skipped), verify
  with the whole model, accept the matching prefix; the emitted tokens equal plain greedy
  decoding.
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
from tests.gpu_util import (check_layer_stages, check_rel, dev, host, same_value, say, stream, v_from_device,
                            v_to_device)
from tests.test_gpu_layer import TINY, DeviceLayer, Model, decode_tokens

pytestmark = pytest.mark.gpu

SMALL = recipes.LayerShape(dim=1024, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn_dim=2816, max_ctx=280)


def run_layer_k_and_check(shape, mix, pos, k, n_slots, layer=0):
    say(f"decode layer x{k} dim={shape.dim} pos={pos}..{pos + k - 1}")
    L = DeviceLayer(shape, mix, layer, n_slots)
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_k_ws_bytes(shp, k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    off = nt.nt_decode_layer_k_ws_offsets(shp, k)
    H0 = np.stack([synth.normal_f32(shape.dim, 3, 900 + t) for t in range(k)])
    h = dev(H0)
    nt.nt_decode_layer_k(L.weights(), shp, pos, k, h.data_ptr(), L.kc.data_ptr(), L.vc.data_ptr(), ws.data_ptr(), wsb,
                         stream())
    torch.cuda.synchronize()
    nq = shape.n_q_heads * shape.head_dim

    def wsf(name, n):
        return ws[off[name]:off[name] + 4 * k * n].view(torch.float32).cpu().numpy().reshape(k, n)

    g_q, g_o, g_h1, g_a = wsf("q", nq), wsf("o", nq), wsf("h1", shape.dim), wsf("a", shape.ffn_dim)
    g_h2 = host(h).reshape(k, shape.dim)
    kc, vc = host(L.kc), v_from_device(host(L.vc), shape.n_kv_heads, shape.max_ctx)
    keep = np.ones(shape.max_ctx, bool)
    keep[pos:pos + k] = False
    assert same_value(kc[:, keep], L.kc_host[:, keep]) and same_value(vc[:, keep], L.vc_host[:, keep])
    worst = {}
    kc_t, vc_t = L.kc_host.copy(), L.vc_host.copy()
    for t in range(k):
        p = pos + t
        g = {"k16": kc[:, p, :].ravel(), "v16": vc[:, p, :].ravel(), "q": g_q[t], "o": g_o[t], "h1": g_h1[t],
             "a": g_a[t], "h2": g_h2[t]}
        st = oracle.decode_layer(L.host, mix, shape, p, H0[t], kc_t, vc_t,
                                 forced={n: g[n] for n in ("k16", "v16", "q", "o", "h1", "a")})
        res = check_layer_stages(st, g, what=f"token {t}")
        for n, v in res.items():
            worst[n] = max(worst.get(n, 0.0), v)
        # the next token's checker sees this token's cache entries, as the GPU wrote them
        kc_t[:, p, :] = kc[:, p, :]
        vc_t[:, p, :] = vc[:, p, :]
    say("  worst " + ", ".join(f"{n} {v:.1e}" for n, v in worst.items()))


@pytest.mark.parametrize("k", [2, 4, 8])
def test_layer_k_70b_q4_k_m(k):
    run_layer_k_and_check(recipes.LLAMA31_70B, recipes.MIX_Q4_K_M, 4096, k, 4096, layer=1)


@pytest.mark.parametrize("mix,pos,k", [
    (recipes.MIX_Q8_0, 250, 8),    # tokens on both sides of the 256-slot split boundary
    (recipes.MIX_Q6_K, 0, 3),      # from an empty cache
    (recipes.MIX_Q4_K_M, 275, 5),  # the last five slots of the cache
    (recipes.MIX_Q5_K_M, 37, 1),
    ({n: synth.Q4_0 for n in recipes.TENSORS}, 100, 7),
])
def test_layer_k_small_shapes(mix, pos, k):
    run_layer_k_and_check(SMALL, mix, pos, k, n_slots=pos)


def test_layer_k_8b_q8_0():
    run_layer_k_and_check(recipes.LLAMA3_8B, recipes.MIX_Q8_0, 1016, 8, 1016)


def _verify(model, kcs, vcs, plan, tokens, pos, st=None, compute=None, copy=None):
    k = len(tokens)
    shp = tg.layer_shape(model.shape)
    wsb = nt.nt_verify_tokens_ws_bytes(shp, k)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(k * model.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(k * model.vocab, dtype=torch.float32, device="cuda")
    tin = torch.tensor(tokens, dtype=torch.int32, device="cuda")
    nxt = torch.full((k,), -1, dtype=torch.int32, device="cuda")
    compute = compute or torch.cuda.Stream()
    copy = copy or torch.cuda.Stream()
    nt.nt_verify_tokens(st, plan, model.head(), pos, k, tin.data_ptr(), nxt.data_ptr(), logits.data_ptr(),
                        h.data_ptr(), ws.data_ptr(), wsb, compute.cuda_stream, copy.cuda_stream)
    torch.cuda.synchronize()
    return ([int(x) for x in host(nxt)], host(h).reshape(k, -1).copy(), host(logits).reshape(k, -1).copy())


@pytest.mark.parametrize("k", [1, 3, 8])
def test_verify_tokens_match_sequential_greedy(k):
    """The greedy picks after each of k given tokens equal sequential greedy decoding; logits
    within tolerance of the checker on the GPU's final hidden states; caches as after k tokens."""
    say(f"verify {k} tokens vs sequential greedy decode")
    m = Model(TINY, recipes.MIX_Q4_K_M, 4, vocab=1000, n_slots=32)
    tok0 = synth.uniform_index(1000, 0, 81)
    seq, hs, lgs, kref, vref, _ = decode_tokens(m, set(), tok0, 32, k)
    inputs = [tok0] + seq[:-1]
    kcs, vcs = m.caches()
    plan, keep = m.plan(kcs, vcs, set())
    nxt, H, LG = _verify(m, kcs, vcs, plan, inputs, 32)
    assert nxt == seq, (nxt, seq)
    for t in range(k):
        n = oracle.rmsnorm(H[t], m.onorm, TINY.eps)
        ref, nrm = oracle.gemv(synth.Q4_K, 1000, TINY.dim, m.out, n)
        check_rel(LG[t], ref, nrm, what=f"logits of token {t}")
        assert ref[nxt[t]] >= ref.max() - 1e-3 * nrm[nxt[t]]
        assert nxt[t] == int(np.argmax(LG[t]))
    # every layer's cache holds the k new slots: the same values as the sequential run's up to
    # rounding (normwise; each entry is judged against the checker in the layer tests)
    for l in range(4):
        for got_c, ref_c in ((host(kcs[l]), kref[l]), (host(vcs[l]), vref[l])):
            a16 = got_c.view(np.float16).astype(np.float64)
            b16 = ref_c.view(np.float16).astype(np.float64)
            rel = np.linalg.norm(a16 - b16) / np.linalg.norm(b16)
            worst = np.unravel_index(np.argmax(np.abs(a16 - b16)), a16.shape)
            say(f"  layer {l}: cache normwise rel diff {rel:.1e}, worst at {worst}: {a16[worst]} vs {b16[worst]}")
            assert rel < 1e-3  # the GEMV tolerance; the two runs differ by fp16 rounding flips


def test_verify_tokens_streamed_equals_resident():
    """Streamed layers in the verify pass (each blob copied once for all tokens) give bit for
    bit what the resident model gives."""
    say("verify pass: streamed vs resident")
    m = Model(TINY, recipes.MIX_Q4_K_M, 4, vocab=1000, n_slots=32)
    toks = [5, 17, 999, 0]
    kcs, vcs = m.caches()
    plan, keep = m.plan(kcs, vcs, set())
    a = _verify(m, kcs, vcs, plan, toks, 32)
    kcs2, vcs2 = m.caches()
    plan2, keep2 = m.plan(kcs2, vcs2, {1, 3})
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), m.lay.nbytes)
    try:
        b = _verify(m, kcs2, vcs2, plan2, toks, 32, st=st)
    finally:
        torch.cuda.synchronize()
        nt.nt_stream_destroy(st)
    assert a[0] == b[0] and same_value(a[1], b[1]) and same_value(a[2], b[2])
    for l in range(4):
        assert same_value(host(kcs[l]), host(kcs2[l])) and same_value(host(vcs[l]), host(vcs2[l]))


def self_speculative_decode(m, tok0, pos0, n_out, k, resident, staging):
    """Greedy self-speculative decoding: the resident layers (the others skipped) draft k - 1
    tokens one by one; the whole model verifies the current token and the drafts in one pass;
    the drafts are accepted while they match the verified picks, and the first differing pick
    (or the pick after the last draft) is emitted too.  Returns the emitted tokens and the
    acceptance counts."""
    kcs, vcs = m.caches()
    streamed = set(range(m.n_layers)) - set(resident)
    full, keep_f = m.plan(kcs, vcs, streamed)
    draft, keep_d = m.plan(kcs, vcs, streamed, skip=streamed)
    shp = tg.layer_shape(m.shape)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(m.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
    dt = torch.zeros(1, dtype=torch.int32, device="cuda")
    compute, copy = torch.cuda.Stream(), torch.cuda.Stream()
    st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), m.lay.nbytes)
    out, accepted = [], []
    cur, pos = tok0, pos0
    try:
        while len(out) < n_out:
            kk = min(k, m.shape.max_ctx - pos)
            drafts = []
            dt.fill_(cur)
            for i in range(kk - 1):  # the draft model: resident layers only, nothing streamed
                nt.nt_decode_token(None, draft, m.head(), pos + i, dt.data_ptr(), logits.data_ptr(), h.data_ptr(),
                                   ws.data_ptr(), wsb, compute.cuda_stream, copy.cuda_stream)
                torch.cuda.synchronize()
                drafts.append(int(host(dt)[0]))
            nxt, _, _ = _verify(m, kcs, vcs, full, [cur] + drafts, pos, st=st, compute=compute, copy=copy)
            n = 0
            while n < len(drafts) and drafts[n] == nxt[n]:
                n += 1
            emitted = nxt[:n + 1]
            out += emitted
            accepted.append(n)
            cur, pos = emitted[-1], pos + n + 1
    finally:
        torch.cuda.synchronize()
        nt.nt_stream_destroy(st)
    return out[:n_out], accepted


def test_self_speculative_decoding_equals_greedy():
    say("self-speculative decoding (resident layers draft, whole model verifies) vs plain greedy")
    m = Model(TINY, recipes.MIX_Q4_K_M, 4, vocab=1000, n_slots=16)
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    tok0 = synth.uniform_index(1000, 0, 82)
    ref = decode_tokens(m, {2, 3}, tok0, 16, 12, staging)[0]
    for k in (2, 4):
        got, acc = self_speculative_decode(m, tok0, 16, 12, k, resident=(0, 1), staging=staging)
        say(f"  k={k}: accepted drafts per step {acc}")
        assert got == ref, (k, got, ref)
