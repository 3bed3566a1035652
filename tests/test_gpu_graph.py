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
