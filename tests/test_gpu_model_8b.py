"""Full-depth parity of the 8B workload the benchmark decodes (MI355X only): the 32-layer
Llama-3-8B-shaped model in Q8_0 with a Q8_0 embedding and 128256 x 4096 LM head, resident, one
greedy token at position 1023 over a 1024-slot fp16 cache (slots below 1023 prefilled).

As for the 70B model: the token is decoded with nt_decode_token, replayed layer by layer with
nt_decode_layer (bit for bit the same final hidden state), every stage of every layer judged
against the checker teacher-forced at the layer boundary, and the LM head element-wise over the
whole vocabulary.  This head is large enough to take the streamed GEMV path, so its fused argmax
(the streamed kernel's logits epilogue) is checked against planted exact ties in other
workgroups as well (ntransformer overview, de.news.hada.io, "Roadmap der Entwicklungsphasen":
Llama 8B in Q8_0; "Architektur und Codestruktur": sampler)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import quantized_weight_streaming_dequant_amd as nt
import synth
from quantized_weight_streaming_dequant_amd import torch_glue as tg
from synth import recipes
from tests.gpu_util import check_layer_stages, check_rel, host, say

pytestmark = pytest.mark.gpu

SHAPE = recipes.LLAMA3_8B
MIX = recipes.MIX_Q8_0
N_LAYERS = 32
POS = 1023
VOCAB = recipes.VOCAB_70B
ROW_BYTES = SHAPE.dim // 32 * 34  # one Q8_0 row of the LM head


@pytest.fixture(scope="module")
def decoded():
    import bench
    nt.load()
    say("8B Q8_0, 32 layers resident: generating the model")
    m = bench.Model70B(torch, nt, tg, MIX, N_LAYERS, range(N_LAYERS), n_prefill=POS, shape=SHAPE, head_fmt=synth.Q8_0,
                       tiles=True)
    plan, keep = m.plan()
    head = m.head()
    shp = tg.layer_shape(SHAPE)
    cs = torch.cuda.current_stream().cuda_stream
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(SHAPE.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(VOCAB, dtype=torch.float32, device="cuda")
    tok = torch.tensor([m.first_token], dtype=torch.int32, device="cuda")
    say(f"  nt_decode_token: token {m.first_token} at pos {POS}")
    nt.nt_decode_token(None, plan, head, POS, tok.data_ptr(), logits.data_ptr(), h.data_ptr(), ws.data_ptr(), wsb,
                       cs, cs, None)
    torch.cuda.synchronize()
    out = {"model": m, "token": int(tok.item()), "h_final": host(h).copy(), "logits": host(logits).copy()}
    say(f"  greedy token {out['token']}; replaying layer by layer")
    off = nt.nt_decode_layer_ws_offsets(shp)
    lws = torch.zeros(nt.nt_decode_layer_ws_bytes(shp), dtype=torch.uint8, device="cuda")
    t0 = torch.tensor([m.first_token], dtype=torch.int32, device="cuda")
    hr = torch.zeros(SHAPE.dim, dtype=torch.float32, device="cuda")
    nt.nt_embed_row(m.embd_fmt, VOCAB, SHAPE.dim, m.embd.data_ptr(), t0.data_ptr(), hr.data_ptr(), cs)
    nq, nkv = SHAPE.n_q_heads * SHAPE.head_dim, SHAPE.n_kv_heads

    def wsf(name, n):
        return lws[off[name]:off[name] + 4 * n].view(torch.float32).cpu().numpy().copy()

    caps = []
    for l in range(N_LAYERS):
        h_in = host(hr).copy()
        nt.nt_decode_layer(m.layer_weights(l), shp, POS, hr.data_ptr(), m.kc[l].data_ptr(), m.vc[l].data_ptr(),
                           lws.data_ptr(), lws.numel(), cs)
        torch.cuda.synchronize()
        k16 = m.kc[l].view(nkv, SHAPE.max_ctx, 128)[:, POS, :].cpu().numpy().view(np.uint16).ravel().copy()
        v16 = m.vc[l].view(nkv, SHAPE.max_ctx // 8, 128, 8)[:, POS // 8, :, POS % 8].cpu().numpy()
        caps.append({"h_in": h_in, "q": wsf("q", nq), "o": wsf("o", nq), "h1": wsf("h1", SHAPE.dim),
                     "a": wsf("a", SHAPE.ffn_dim), "h2": host(hr).copy(), "k16": k16,
                     "v16": np.ascontiguousarray(v16).view(np.uint16).ravel().copy()})
    out["caps"] = caps
    out["h_replay"] = host(hr).copy()
    yield out
    del m
    torch.cuda.empty_cache()


def test_replay_matches_the_token_step(decoded):
    assert np.array_equal(decoded["h_replay"], decoded["h_final"])


def test_every_layer_teacher_forced(decoded):
    worst = {}
    for l in range(N_LAYERS):
        c = decoded["caps"][l]
        w = recipes.layer_arrays(SHAPE, MIX, l)
        kc = recipes.kv_cache_array(SHAPE, l, "k", POS)
        vc = recipes.kv_cache_array(SHAPE, l, "v", POS)
        st = oracle.decode_layer(w, MIX, SHAPE, POS, c["h_in"], kc, vc,
                                 forced={k: c[k] for k in ("k16", "v16", "q", "o", "h1", "a")})
        res = check_layer_stages(st, c, what=f"layer {l}")
        for k, v in res.items():
            worst[k] = max(worst.get(k, 0.0), v)
    say("  32 layers: worst " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))


def test_lm_head_full_vocabulary_and_greedy_pick(decoded):
    m = decoded["model"]
    n = oracle.rmsnorm(decoded["h_final"], host(m.onorm), SHAPE.eps)
    ref, nrm = oracle.gemv(synth.Q8_0, VOCAB, SHAPE.dim, host(m.out), n)
    worst = check_rel(decoded["logits"], ref, nrm, what="logits")
    tok = decoded["token"]
    assert tok == int(np.argmax(decoded["logits"]))
    assert ref[tok] >= ref.max() - 1e-3 * nrm[tok]
    say(f"  logits worst rel {worst:.1e}; token {tok} (checker's argmax {int(np.argmax(ref))})")


def test_streamed_head_argmax_planted_exact_ties(decoded):
    """Copies of the winning row far below it, at its neighbour and at the last row: identical
    rows give identical logits, and the streamed head's pick is the lowest tied index."""
    m = decoded["model"]
    b = decoded["token"]
    out2 = m.out.clone()
    rows = out2.view(VOCAB, ROW_BYTES)
    ties = sorted({(b + 40000) % VOCAB, b ^ 1, (b + 90001) % VOCAB, VOCAB - 1} - {b})
    for j in ties:
        rows[j] = rows[b]
    h = torch.from_numpy(decoded["h_final"]).cuda()
    logits = torch.zeros(VOCAB, dtype=torch.float32, device="cuda")
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nt.NT_LM_HEAD_WS_BYTES, dtype=torch.uint8, device="cuda")
    nt.nt_lm_head(synth.Q8_0, VOCAB, SHAPE.dim, out2.data_ptr(), m.onorm.data_ptr(), SHAPE.eps, h.data_ptr(),
                  logits.data_ptr(), tok.data_ptr(), ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    lg = host(logits)
    for j in ties:
        assert lg[j] == lg[b], (j, lg[j], lg[b])
    t = int(tok.item())
    assert t == min(ties + [b]) == int(np.argmax(lg)), (t, ties, b)
    say(f"  winner {b}, tied copies {ties}: pick {t}")
    del out2
