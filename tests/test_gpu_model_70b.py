"""Full-depth parity of the benchmarked workload (MI355X only): the 80-layer
Llama-3.1-70B-shaped model in the Q4_K_M mix, resident, one greedy token at position 4096
after a 4096-slot fp16 cache, with its 128256 x 8192 LM head; as in the benchmark, the Q4_K
matrices and the LM head are held in the library's tiled layout (nt_repack, NT_Q4_KT), and the
checker reads the same weights in Q4_K's block order.

The token is decoded with nt_decode_token, the call the benchmark times, then replayed layer
by layer with nt_decode_layer (the same kernels: the replay must reach the same final hidden
state bit for bit) so that every stage of every layer can be captured and judged against the
checker, teacher-forced at the layer boundary (each layer's checker run starts from the GPU's
input to that layer).  The LM head is judged element-wise over the whole vocabulary, the greedy
pick by the acceptance rule (its checker logit within 1e-3 of the normaliser of the maximum),
and the fused argmax against planted exact ties and near-ties between rows that sit in
different workgroups (ntransformer overview, de.news.hada.io, "Architektur und Codestruktur":
sampler and engine; "Roadmap der Entwicklungsphasen": the 70B model).
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
from tests.gpu_util import check_layer_stages, check_rel, host, say

pytestmark = pytest.mark.gpu

SHAPE = recipes.LLAMA31_70B
MIX = recipes.MIX_Q4_K_M
N_LAYERS = 80
POS = 4096
VOCAB = recipes.VOCAB_70B
ROW_BYTES = SHAPE.dim // 256 * 144  # one Q4_K row of the LM head


@pytest.fixture(scope="module")
def decoded():
    import bench
    nt.load()
    say("70B Q4_K_M, 80 layers resident: generating the model")
    m = bench.Model70B(torch, nt, tg, MIX, N_LAYERS, range(N_LAYERS), tiles=True)
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
    out = {"model": m, "tok0": m.first_token, "token": int(tok.item()), "h_final": host(h).copy(),
           "logits": host(logits).copy()}
    say(f"  greedy token {out['token']}; replaying layer by layer")
    # the replay: embedding row, then every layer with nt_decode_layer, every stage captured
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
        # V cache in groups of 8 slots: [n_kv][max_ctx / 8][128][8]
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


@pytest.mark.parametrize("first", [0, 20, 40, 60])
def test_every_layer_teacher_forced(decoded, first):
    worst = {}
    for l in range(first, first + 20):
        c = decoded["caps"][l]
        w = recipes.layer_arrays(SHAPE, MIX, l)
        kc = recipes.kv_cache_array(SHAPE, l, "k", POS)
        vc = recipes.kv_cache_array(SHAPE, l, "v", POS)
        st = oracle.decode_layer(w, MIX, SHAPE, POS, c["h_in"], kc, vc,
                                 forced={k: c[k] for k in ("k16", "v16", "q", "o", "h1", "a")})
        res = check_layer_stages(st, c, what=f"layer {l}")
        for k, v in res.items():
            worst[k] = max(worst.get(k, 0.0), v)
    say(f"  layers {first}..{first + 19}: worst " + ", ".join(f"{k} {v:.1e}" for k, v in worst.items()))


def _head_ref(decoded, out_host, rows=None):
    m = decoded["model"]
    n = oracle.rmsnorm(decoded["h_final"], host(m.onorm), SHAPE.eps)
    return oracle.gemv(synth.Q4_K, VOCAB, SHAPE.dim, out_host, n, row_idx=rows)


def test_lm_head_full_vocabulary_and_greedy_pick(decoded):
    m = decoded["model"]
    out_host = host(m.out)
    ref, nrm = _head_ref(decoded, out_host)
    worst = check_rel(decoded["logits"], ref, nrm, what="logits")
    tok = decoded["token"]
    # the fused argmax is the first index of the largest stored logit
    assert tok == int(np.argmax(decoded["logits"]))
    # acceptance of the greedy pick: its exact logit is within the tolerance of the maximum
    assert ref[tok] >= ref.max() - 1e-3 * nrm[tok]
    say(f"  logits worst rel {worst:.1e}; token {tok} (checker's argmax {int(np.argmax(ref))})")


def _lm_head(decoded, out_dev):
    m = decoded["model"]
    h = torch.from_numpy(decoded["h_final"]).cuda()
    logits = torch.zeros(VOCAB, dtype=torch.float32, device="cuda")
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nt.NT_LM_HEAD_WS_BYTES, dtype=torch.uint8, device="cuda")
    nt.nt_lm_head(synth.Q4_K, VOCAB, SHAPE.dim, out_dev.data_ptr(), m.onorm.data_ptr(), SHAPE.eps, h.data_ptr(),
                  logits.data_ptr(), tok.data_ptr(), ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return int(tok.item()), host(logits).copy()


def test_lm_head_entry_matches_the_token_step(decoded):
    tok, logits = _lm_head(decoded, decoded["model"].out)
    assert tok == decoded["token"] and np.array_equal(logits, decoded["logits"])


def test_fused_argmax_planted_exact_ties(decoded):
    """Copies of the winning row at a lower index far away, at its group neighbour and near the
    end: identical rows give identical logits, and the pick is the lowest tied index."""
    b = decoded["token"]
    out2 = decoded["model"].out.clone()
    rows = out2.view(VOCAB, ROW_BYTES)
    ties = sorted({(b + 40000) % VOCAB, b ^ 1, (b + 90001) % VOCAB, VOCAB - 1} - {b})
    for j in ties:
        rows[j] = rows[b]
    tok, logits = _lm_head(decoded, out2)
    for j in ties:
        assert logits[j] == logits[b], (j, logits[j], logits[b])
    assert tok == min(ties + [b]), (tok, ties, b)
    assert tok == int(np.argmax(logits))
    del out2


def test_fused_argmax_planted_near_ties(decoded):
    """Copies of the winning row with one 4-bit code moved by one step, at a column chosen so
    that the copy's exact logit differs from the winner's by 8 to 64 fp32 units of the winner's
    logit, once upward and once downward, at indices in other workgroups: the stored logits
    order the three rows as the checker does, and the pick is the first index of the largest."""
    m = decoded["model"]
    b = decoded["token"]
    n = oracle.rmsnorm(decoded["h_final"], host(m.onorm), SHAPE.eps)
    out_host = host(m.out).reshape(VOCAB, ROW_BYTES).copy()
    row_b = out_host[b].copy()
    y_b, _ = oracle.gemv(synth.Q4_K, 1, SHAPE.dim, row_b, n)
    ulp = float(np.spacing(np.float32(y_b[0])))
    targets = [((b + 50000) % VOCAB, +1), ((b + 70001) % VOCAB, -1)]
    # candidate columns: |x| near the size at which one code step moves the logit ~16 units
    # (a weight step d sc is ~0.16 for these scale distributions)
    order = np.argsort(np.abs(np.abs(n) - 16 * ulp / 0.16))
    planted = []
    for j, want in targets:
        done = False
        for c in order[:512]:
            sb, i = divmod(int(c), 256)
            sub, g, l = i // 32, i // 64, i % 32
            byte = sb * 144 + 16 + 32 * g + l
            shift = 4 * (sub % 2)
            q = (int(row_b[byte]) >> shift) & 15
            step = want if n[c] > 0 else -want  # the code step that moves the logit the wanted way
            if not 0 <= q + step <= 15:
                continue
            row = row_b.copy()
            row[byte] = (int(row[byte]) & ~(15 << shift) & 0xFF) | ((q + step) << shift)
            y, _ = oracle.gemv(synth.Q4_K, 1, SHAPE.dim, row, n)
            if 8 * ulp <= (y[0] - y_b[0]) * want <= 64 * ulp:
                out_host[j] = row
                planted.append((j, float(y[0] - y_b[0])))
                done = True
                break
        assert done, f"no near-tie could be planted at row {j}"
    out2 = torch.from_numpy(out_host.reshape(-1)).cuda()
    tok, logits = _lm_head(decoded, out2)
    rows = [b] + [j for j, _ in planted]
    ref, nrm = oracle.gemv(synth.Q4_K, VOCAB, SHAPE.dim, out_host.reshape(-1), n, row_idx=rows)
    check_rel(logits[rows], ref, nrm, what="planted rows")
    j_up, j_down = planted[0][0], planted[1][0]
    assert logits[j_down] < logits[b] < logits[j_up], [float(logits[r]) for r in rows]
    assert tok == int(np.argmax(logits)) == j_up
    say(f"  winner {b}, planted {planted} ({ulp:.1e} per fp32 unit): logits {[float(logits[r]) for r in rows]}, "
        f"pick {tok}")
    del out2
