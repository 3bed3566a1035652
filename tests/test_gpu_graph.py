"""The greedy token step is capturable into a HIP graph (MI355X only): nt_decode_token only
enqueues kernels on the given stream (no allocation, synchronisation, memset or copy), so a
graph captured around one call replays, replay after replay, the bytes the call gives when
enqueued directly.  Each replay follows eager work of the program's own and a synchronisation,
and every replay is checked (hipMemsetAsync nodes, which this path must not contain, have been
seen to go wrong on replays after the first)."""
from __future__ import annotations

import pytest
import torch

import quantized_weight_streaming_dequant_amd as nt
from quantized_weight_streaming_dequant_amd import torch_glue as tg
from synth import recipes
from tests.gpu_util import say
from tests.test_gpu_layer import TINY, Model

pytestmark = pytest.mark.gpu


def test_token_step_graph_replay_bit_identical():
    say("token step: HIP graph replay vs direct enqueue (3 layers, vocab 500, pos 20)")
    m = Model(TINY, recipes.MIX_Q4_K_M, 3, vocab=500, n_slots=20)
    kcs, vcs = m.caches()
    plan, keep = m.plan(kcs, vcs, set())
    head = m.head()
    shp = tg.layer_shape(TINY)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(TINY.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(500, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    pos, tok0 = 20, 123
    s = torch.cuda.Stream()

    def step():
        r = nt.nt_decode_token(None, plan, head, pos, tok.data_ptr(), logits.data_ptr(), h.data_ptr(), ws.data_ptr(),
                               wsb, s.cuda_stream, s.cuda_stream, None)
        assert r == 0, nt.nt_last_error()

    def reset():  # on the default stream, then synchronised
        tok.fill_(tok0)
        h.fill_(3.0)
        logits.fill_(-1.0)
        torch.cuda.synchronize()

    def state():
        return [tok.clone(), h.clone(), logits.clone()] + [k.clone() for k in kcs] + [v.clone() for v in vcs]

    reset()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    ref = state()
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        x = torch.randn(1 << 20, device="cuda")  # eager work between the replays
        (x * x).sum().item()
        g.replay()
        torch.cuda.synchronize()
        got = state()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
    say(f"  token {int(ref[0].item())}; three replays bit-identical to the direct call")


def test_noalloc_layer_graph_replay_bit_identical():
    """nt_decode_layer_noalloc is meant for callers under graph capture: captured once (after a
    first direct call has looked up its static workspace) and replayed three times, it gives the
    direct call's h, K and V bit for bit."""
    from tests.gpu_util import dev, v_to_device
    shape = recipes.LayerShape(dim=1024, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn_dim=2816, max_ctx=96)
    mix, pos = recipes.MIX_Q4_K_M, 50
    say(f"noalloc layer: HIP graph replay vs direct call (dim {shape.dim}, pos {pos})")
    w = recipes.layer_arrays(shape, mix, 0)
    d = {k: dev(v) for k, v in w.items()}
    lw = tg.layer_weights([mix[n] for n in recipes.TENSORS], [d[n] for n in recipes.TENSORS], d["attn_norm"],
                          d["ffn_norm"])
    kc = dev(recipes.kv_cache_array(shape, 0, "k", pos))
    vc = dev(v_to_device(recipes.kv_cache_array(shape, 0, "v", pos), shape.n_kv_heads, shape.max_ctx))
    h0 = dev(recipes.hidden_input(shape.dim))
    h = h0.clone()
    shp = tg.layer_shape(shape)
    s = torch.cuda.Stream()

    def call():
        nt.nt_decode_layer_noalloc(lw, shp, pos, h.data_ptr(), kc.data_ptr(), vc.data_ptr(), s.cuda_stream)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    ref = [h.clone(), kc.clone(), vc.clone()]
    h.copy_(h0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        h.copy_(h0)
        x = torch.randn(1 << 20, device="cuda")  # eager work between the replays
        (x * x).sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((h, kc, vc), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep} differs"
    say("  three replays bit-identical to the direct call")
