"""nt_decode_layer_noalloc, the decode layer for callers that cannot allocate (its workspace is
a static device array), against nt_decode_layer with a caller workspace (MI355X only), through
the C ABI: two calls in a row on fresh copies of the same inputs, the second with a smaller
layer, each bit-identical to the caller-workspace entry (the same kernels); its stage outputs
are left in the static array, so the second call also shows that nothing of the first call's
contents leaks into it."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import quantized_weight_streaming_dequant_amd as nt
from quantized_weight_streaming_dequant_amd import torch_glue as tg
from synth import recipes
from tests.gpu_util import dev, host, same_value, say, stream, v_to_device

pytestmark = pytest.mark.gpu

SMALL = recipes.LayerShape(dim=1024, n_q_heads=16, n_kv_heads=4, head_dim=128, ffn_dim=2816, max_ctx=96)


def _run(shape, mix, pos, n_slots, layer, noalloc):
    w = recipes.layer_arrays(shape, mix, layer)
    d = {k: dev(v) for k, v in w.items()}
    lw = tg.layer_weights([mix[n] for n in recipes.TENSORS], [d[n] for n in recipes.TENSORS], d["attn_norm"],
                          d["ffn_norm"])
    kc = dev(recipes.kv_cache_array(shape, layer, "k", n_slots))
    vc = dev(v_to_device(recipes.kv_cache_array(shape, layer, "v", n_slots), shape.n_kv_heads, shape.max_ctx))
    h = dev(recipes.hidden_input(shape.dim))
    shp = tg.layer_shape(shape)
    if noalloc:
        nt.nt_decode_layer_noalloc(lw, shp, pos, h.data_ptr(), kc.data_ptr(), vc.data_ptr(), stream())
    else:
        wsb = nt.nt_decode_layer_ws_bytes(shp)
        ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")
        nt.nt_decode_layer(lw, shp, pos, h.data_ptr(), kc.data_ptr(), vc.data_ptr(), ws.data_ptr(), wsb, stream())
    torch.cuda.synchronize()
    return host(h).copy(), host(kc).copy(), host(vc).copy()


@pytest.mark.parametrize("shape,mix,pos,n_slots,layer", [
    (recipes.LLAMA31_70B, recipes.MIX_Q4_K_M, 4200, 4096, 2),  # first call: 70B shape, 17 attention splits
    (SMALL, recipes.MIX_Q8_0, 50, 96, 1),                        # second call: a smaller layer
])
def test_noalloc_layer_matches_caller_workspace(shape, mix, pos, n_slots, layer):
    say(f"noalloc decode layer dim={shape.dim} pos={pos} vs caller workspace")
    a = _run(shape, mix, pos, n_slots, layer, noalloc=False)
    b = _run(shape, mix, pos, n_slots, layer, noalloc=True)
    for x, y in zip(a, b):
        assert same_value(x, y)
    assert np.all(np.isfinite(b[0]))


def test_noalloc_rejects_a_workspace_past_the_static_size():
    shape = recipes.LayerShape(dim=8192, n_q_heads=64, n_kv_heads=8, head_dim=128, ffn_dim=28672, max_ctx=65536)
    shp = tg.layer_shape(shape)
    assert nt.nt_decode_layer_ws_bytes(shp) > nt.NT_NOALLOC_WS_BYTES
    with pytest.raises(nt.NtError) as ei:
        nt.nt_decode_layer_noalloc(nt.LayerWeights(), shp, 0, 256, 256, 256, stream())
    assert ei.value.code == nt.NT_ESHAPE and "static" in nt.last_error()
