#!/usr/bin/env python3
"""Benchmark of the batch-1 quantized decode path on one MI355X.

Default workload: an 80-layer Llama-3.1-70B-shaped model (hidden 8192, 64/8 heads of 128,
FFN 28672, vocabulary 128256) with synthetic weights in the Q4_K_M mix (Q4_K, with Q6_K
for attn_v and ffn_down), all resident in HBM, greedy decode of one token per step after
a 4096-slot synthetic fp16 KV cache.  A step is one whole token: embedding row, 80
decode layers, final norm, LM head and argmax, every kernel in libnt.so.

Prints one JSON line.  Other workloads (--config) print their own line for measurement
runs: 1 = Q8_0 GEMV 4096x4096, 2 = one Llama-3-8B-shaped Q8_0 layer, 3 = the 70B GEMV
shapes in Q4_K, Q6_K, Q5_K, F16, F32 and tiled Q4_K and Q5_K, 5 = the 70B Q6_K model with 54 layers streamed from pinned
host memory, 6 = the k-token GEMM (k = 1, 2, 4, 8) at the 70B shapes, 7 = the 70B model with
cosine-based layer skip (--skip layers, default 20 of 80), 8 = 70B Q6_K layers read from a file
(--file-layers, default 8) through page-locked bounce buffers, 9 = the self-speculative
verification pass (k-token layer and whole-model verify at k = 2, 4, 8) at the 70B shape, 10 =
self-speculative decoding over the streamed 70B Q6_K model (resident layers draft, --spec-k).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0



def v_to_device_layout(torch, v, n_kv, max_ctx, hd=128):
    """[n_kv][max_ctx][hd] fp16 V cache -> the library's [n_kv][max_ctx/8][hd][8] (device copy)."""
    return v.view(n_kv, max_ctx // 8, 8, hd).transpose(2, 3).contiguous().view(-1)

def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
    p.add_argument("--spec-k", type=int, default=4, help="tokens per verify pass in --config 10")
    p.add_argument("--skip", type=int, default=20, help="layers to skip in --config 7")
    p.add_argument("--file-layers", type=int, default=8, help="layers read from a file in --config 8")
    p.add_argument("--read-threads", type=int, default=8, help="reader threads per blob in --config 8")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip the GEMV and 8B-layer measurements of the default run")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--layers", type=int, default=80, help="layers of the 70B model (measurement runs only)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (the reference for HBM byte counters)")
    return p.parse_args()


# ----------------------------------------------------------------------------- helpers

ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_gate_up_q4k_70b_traffic.txt")
TRAFFIC_SOURCES = [os.path.join(ROOT, "quantized_weight_streaming_dequant_amd", "csrc", f)
                   for f in ("gemv.hip", "gemv.h", "common.h")]


def sources_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a plain copy of
    known size), or None when there is none or the kernel sources changed since."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            for line in fh:
                if line.startswith("TRAFFIC_JSON "):
                    d = json.loads(line[len("TRAFFIC_JSON "):])
                    if d.get("sources_sha256") == sources_digest():
                        return d["hbm_bytes_per_launch"]
    except OSError:
        pass
    return None


def copy_calibration(torch):
    """A plain device copy of 1 GiB, ten times: the kernel whose byte counters are known."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes": n, "copies": 10}


def read_probe(torch, nt, nbytes=4 << 30, reps=20):
    """The achievable HBM read rate: nt_read_probe (plain 16-byte loads over a buffer far
    larger than the 256 MB last-level cache), HIP events around `reps` back-to-back calls."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cs = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        nt.nt_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), cs)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        nt.nt_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), cs)
    ev1.record()
    ev1.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / reps
    del buf
    return {"GBps": nbytes / (us * 1e-6) / 1e9, "bytes": nbytes, "avg_us": us, "reps": reps,
            "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "kernel": "nt_read_probe: 16-byte nontemporal loads, 2 in flight per thread, 32 workgroups of 256 per CU"}


def host_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))


def timed_class(nt, torch, kclass, run, nbytes_per_launch):
    """Average duration of one kernel class over the launches `run` makes, timed with HIP events
    recorded around each launch on its stream."""
    nt.nt_timing_begin(kclass, 1 << 20)
    run()
    torch.cuda.synchronize()
    n, ms = nt.nt_timing_end()
    avg_ms = ms / max(n, 1)
    return {"launches": n, "avg_us": avg_ms * 1e3, "GBps": nbytes_per_launch / (avg_ms * 1e-3) / 1e9 if n else None}


class Model70B:
    """80 layer blobs + embedding + LM head + caches, generated layer by layer on the host
    (pinned staging) and copied into HBM (another shape, such as the 8B one, by argument)."""

    def __init__(self, torch, nt, tg, mix, n_layers, resident_layers, n_prefill=4096, seed=0, shape=None,
                 head_fmt=None, tiles=False):
        import synth
        from synth import recipes
        self.torch, self.nt, self.tg = torch, nt, tg
        self.shape = recipes.LLAMA31_70B if shape is None else shape
        self.mix = mix
        # tiles: the resident layers' Q4_K and Q8_0 matrices and such an LM head rearranged on the
        # device into the GEMV's tiled layouts (nt_repack: Q4_KT, Q8_0T); the same weights
        self.tiles = tiles
        tiled_fmt = {synth.Q4_K: synth.Q4_KT, synth.Q8_0: synth.Q8_0T, synth.Q5_K: synth.Q5_KT}
        self.fmts = {n: (tiled_fmt.get(mix[n], mix[n]) if tiles else mix[n]) for n in recipes.TENSORS}
        self.n_layers = n_layers
        self.vocab = recipes.VOCAB_70B
        self.lay = recipes.blob_layout(self.shape, mix)
        self.resident = set(resident_layers)
        shp = self.shape
        t0 = time.time()
        stage = [torch.empty(self.lay.nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        done = [None, None]
        copy_stream = torch.cuda.Stream()
        self.dev_blobs, self.host_blobs = {}, {}
        for l in range(n_layers):
            if l in self.resident:
                b = l % 2
                hb = stage[b]
                if done[b] is not None:
                    done[b].synchronize()  # the copy that last read this staging buffer is done
                recipes.fill_layer_blob(hb.data_ptr(), shp, mix, l, seed, self.lay)
                d = torch.empty(self.lay.nbytes, dtype=torch.uint8, device="cuda")
                copy_stream.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(copy_stream):
                    d.copy_(hb, non_blocking=True)
                    done[b] = torch.cuda.Event()
                    done[b].record(copy_stream)
                self.dev_blobs[l] = d
            else:
                hb = torch.empty(self.lay.nbytes, dtype=torch.uint8, pin_memory=True)
                recipes.fill_layer_blob(hb.data_ptr(), shp, mix, l, seed, self.lay)
                self.host_blobs[l] = hb
            if l % 10 == 9:
                log(f"  generated layer {l + 1}/{n_layers} ({time.time() - t0:.1f}s)")
        copy_stream.synchronize()
        del stage
        tiled = [n for n in recipes.TENSORS if self.fmts[n] != mix[n]]
        if tiled and self.resident:
            nbytes = {n: synth.matrix_bytes(mix[n], *self.shape.matrix_shape(n)) for n in tiled}
            scratch = torch.empty(max(nbytes.values()), dtype=torch.uint8, device="cuda")
            cs = torch.cuda.current_stream().cuda_stream
            for l in self.resident:
                for n in tiled:
                    rows, cols = self.shape.matrix_shape(n)
                    o, nb = self.lay.offsets[n], nbytes[n]
                    nt.nt_repack(self.fmts[n], rows, cols, self.dev_blobs[l][o:].data_ptr(), scratch.data_ptr(), cs)
                    self.dev_blobs[l][o:o + nb].copy_(scratch[:nb])
            torch.cuda.synchronize()
            del scratch
        # KV caches per layer, slots < n_prefill ~ N(0,1): K as [n_kv][max_ctx][128] fp16,
        # V regrouped on the device into the library's [n_kv][max_ctx/8][128][8]
        cache_elems = shp.n_kv_heads * shp.max_ctx * shp.head_dim
        self.kc, self.vc = [], []
        kv_host = torch.empty(cache_elems, dtype=torch.int16, pin_memory=True)
        for l in range(n_layers):
            for which, lst in (("k", self.kc), ("v", self.vc)):
                kv_host.zero_()
                recipes.kv_cache_fill(kv_host.data_ptr(), shp, l, which, n_prefill, seed)
                d = kv_host.cuda()
                if which == "v":
                    d = v_to_device_layout(torch, d, shp.n_kv_heads, shp.max_ctx)
                lst.append(d)
        # head
        embd_fmt = out_fmt = head_fmt if head_fmt is not None else (synth.Q4_K if mix["q"] == synth.Q4_K else synth.Q6_K)
        self.embd_fmt, self.out_fmt = embd_fmt, out_fmt
        eb = synth.matrix_bytes(embd_fmt, self.vocab, shp.dim)
        hb = torch.empty(eb, dtype=torch.uint8, pin_memory=True)
        synth.fill_blocks(hb.data_ptr(), embd_fmt, eb // synth.BLOCK_BYTES[embd_fmt], seed,
                          recipes.stream_id(recipes.GLOBAL_LAYER, recipes.GID_TOKEN_EMBD))
        self.embd = hb.cuda()
        synth.fill_blocks(hb.data_ptr(), out_fmt, eb // synth.BLOCK_BYTES[out_fmt], seed,
                          recipes.stream_id(recipes.GLOBAL_LAYER, recipes.GID_OUTPUT))
        self.out = hb.cuda()
        del hb
        # the LM head the decode reads (self.out stays in Q4_K's block order for the checker)
        self.head_fmt, self.head_out = out_fmt, self.out
        if tiles and out_fmt in tiled_fmt:
            self.head_fmt, self.head_out = tiled_fmt[out_fmt], torch.empty_like(self.out)
            nt.nt_repack(self.head_fmt, self.vocab, shp.dim, self.out.data_ptr(), self.head_out.data_ptr(),
                         torch.cuda.current_stream().cuda_stream)
        self.onorm = torch.from_numpy(synth.uniform_f32(shp.dim, seed, recipes.stream_id(recipes.GLOBAL_LAYER,
                                                                                          recipes.GID_OUTPUT_NORM),
                                                        0.9, 1.1)).cuda()
        self.first_token = recipes.first_token(self.vocab, seed)
        torch.cuda.synchronize()
        log(f"  model ready in {time.time() - t0:.1f}s")

    def plan(self, skip=()):
        from synth import recipes
        tg, nt = self.tg, self.nt
        shp = tg.layer_shape(self.shape)
        lay = tg.layer_layout(self.lay.offset_list(), [self.fmts[n] for n in recipes.TENSORS], self.lay.nbytes)
        ents = []
        for l in range(self.n_layers):
            if l in self.resident:
                ents.append((self.dev_blobs[l].data_ptr(), True, self.kc[l].data_ptr(), self.vc[l].data_ptr()))
            else:
                ents.append((self.host_blobs[l].data_ptr(), False, self.kc[l].data_ptr(), self.vc[l].data_ptr()))
        return tg.model_plan(shp, lay, ents, skip)

    def layer_weights(self, l):
        """nt_layer_weights of resident layer l (pointers into its blob)."""
        from synth import recipes
        blob = self.dev_blobs[l]
        off = self.lay.offsets
        mats = [blob[off[n]:] for n in recipes.TENSORS]
        return self.tg.layer_weights([self.fmts[n] for n in recipes.TENSORS], mats,
                                     blob[off["attn_norm"]:].view(self.torch.float32),
                                     blob[off["ffn_norm"]:].view(self.torch.float32))

    def head(self):
        return self.nt.ModelHead(self.embd_fmt, self.embd.data_ptr(), self.vocab, self.onorm.data_ptr(), self.head_fmt,
                                 self.head_out.data_ptr())


def token_bytes_70b(mix, n_layers, pos, vocab=128256):
    """Algorithmic HBM bytes of one decode token at position pos: every weight once, the
    embedding row, the KV slots read, the new K/V written, and the activations."""
    import synth
    from synth import recipes
    shp = recipes.LLAMA31_70B
    w = n_layers * recipes.layer_weight_bytes(shp, mix)
    head_fmt = synth.Q4_K if mix["q"] == synth.Q4_K else synth.Q6_K
    lm = synth.matrix_bytes(head_fmt, vocab, shp.dim)
    embd_row = lm // vocab
    kv_read = n_layers * 2 * shp.n_kv_heads * (pos + 1) * shp.head_dim * 2
    kv_write = n_layers * 2 * shp.n_kv_heads * shp.head_dim * 2
    gains = n_layers * 2 * shp.dim * 4 + shp.dim * 4
    nq = shp.n_q_heads * shp.head_dim
    # per layer: h read by 2 norm prologues + 2 residuals, q/o/a written and read, h written twice
    acts = n_layers * 4 * (4 * shp.dim + 2 * nq + 2 * nq + 2 * shp.ffn_dim + 2 * shp.dim) + 4 * vocab
    return w + lm + embd_row + kv_read + kv_write + gains + acts


def ffn_up_bytes(mix, shape):
    import synth
    rows, cols = shape.ffn_dim, shape.dim
    return 2 * synth.matrix_bytes(mix["gate"], rows, cols) + 4 * (2 * cols + rows)


def _oracle_token_sample(mix, target_s, max_layers=80, head_rows=8192):
    """Time the checker on whole 70B layers (pos 4096) until target_s of work, and on head_rows
    LM-head rows; returns (seconds per 80-layer token, layers timed, rows, seconds of work)."""
    import oracle
    import synth
    from synth import recipes
    shp = recipes.LLAMA31_70B
    t_layers, n = 0.0, 0
    h = recipes.hidden_input(shp.dim)
    while n < max_layers and (n == 0 or t_layers < 0.8 * target_s):
        w = recipes.layer_arrays(shp, mix, n)
        kc = recipes.kv_cache_array(shp, n, "k", 4096)
        vc = recipes.kv_cache_array(shp, n, "v", 4096)
        t = time.time()
        st = oracle.decode_layer(w, mix, shp, 4096, h, kc, vc)
        t_layers += time.time() - t
        h = st["h2"]
        n += 1
    head_fmt = synth.Q4_K if mix["q"] == synth.Q4_K else synth.Q6_K
    out = synth.quant_rows(head_fmt, shp.dim, range(head_rows), 0,
                           recipes.stream_id(recipes.GLOBAL_LAYER, recipes.GID_OUTPUT))
    t = time.time()
    oracle.gemv(head_fmt, head_rows, shp.dim, out, oracle.rmsnorm(h, np.ones(shp.dim), shp.eps))
    t_rows = time.time() - t
    s_per_tok = 80 * (t_layers / n) + t_rows * (128256 / head_rows)
    return s_per_tok, n, head_rows, t_layers + t_rows


def cpu_baseline_extras():
    """The checker on the metric's other halves, whole: the Q8_0 4096 x 4096 GEMV (config 1) and
    one Llama-3-8B-shape Q8_0 layer at pos 1023 (config 2), with every host thread and with one."""
    import oracle
    import synth
    from synth import recipes
    cores = host_threads()
    blocks = synth.quant_matrix(synth.Q8_0, 4096, 4096, 0, 5000)
    x = synth.normal_f32(4096, 0, 999)
    gbytes = synth.matrix_bytes(synth.Q8_0, 4096, 4096) + 4 * 2 * 4096
    shp = recipes.LLAMA3_8B
    w = recipes.layer_arrays(shp, recipes.MIX_Q8_0, 0)
    kc = recipes.kv_cache_array(shp, 0, "k", 1024)
    vc = recipes.kv_cache_array(shp, 0, "v", 1024)
    h = recipes.hidden_input(shp.dim)
    lbytes = sum(synth.matrix_bytes(synth.Q8_0, *shp.matrix_shape(n)) for n in recipes.TENSORS)

    def timed(fn, min_s):
        n, t = 0, time.time()
        while n == 0 or time.time() - t < min_s:
            fn()
            n += 1
        return (time.time() - t) / n

    out = {}
    for label, threads in (("all", None), ("one_thread", 1)):
        old = oracle.set_threads(threads) if threads else None
        try:
            tg_ = timed(lambda: oracle.gemv(synth.Q8_0, 4096, 4096, blocks, x), 0.3)
            tl = timed(lambda: oracle.decode_layer(w, recipes.MIX_Q8_0, shp, 1023, h, kc, vc), 0.5)
        finally:
            if threads:
                oracle.set_threads(old)
        out[label] = {"cores": cores if threads is None else 1,
                      "gemv_q8_0_4096x4096": {"seconds": tg_, "GBps": gbytes / tg_ / 1e9},
                      "layer_8b_q8_0": {"seconds": tl, "GBps": lbytes / tl / 1e9}}
    out["kind"] = "oracle"
    out["sample"] = "the Q8_0 4096x4096 GEMV and one 8B Q8_0 layer at pos 1023 (1024 keys), whole, fp64"
    return out


def cpu_baseline_70b(mix, target_s):
    """The checker (fp64, OpenMP) on a bounded sample of one decode token, scaled to one 80-layer
    token: with every host thread (whole layers until target_s of work, plus 8192 LM-head rows),
    then with one thread (one layer and 1024 rows)."""
    import oracle
    cores = host_threads()
    s_all, n, rows, work = _oracle_token_sample(mix, target_s)
    old = oracle.set_threads(1)
    try:
        s_one, n1, rows1, work1 = _oracle_token_sample(mix, target_s, max_layers=1, head_rows=1024)
    finally:
        oracle.set_threads(old)
    return {"value": 1.0 / s_all, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of 80 decode layers (70B shape, pos 4096) and {rows} of 128256 LM-head rows, "
                      f"fp64, scaled to one token ({work:.1f} s of CPU work)",
            "one_thread": {"value": 1.0 / s_one, "unit": "tok/s", "cores": 1,
                           "sample": f"{n1} decode layer and {rows1} LM-head rows, scaled to one token "
                                     f"({work1:.1f} s of CPU work)"}}


def metric_extras(torch, nt, tg):
    """The GEMV and 8B halves of the metric, measured in the default run: the Q8_0 4096x4096
    GEMV, the 70B GEMV shapes in Q4_K, Q6_K and the tiled Q4_K layout (rotating weight copies past the 256 MB
    last-level cache, HIP events around back-to-back launches) and one Llama-3-8B-shaped
    Q8_0 layer with its derived tokens/s."""
    import synth
    keys = ("rows", "cols", "format", "avg_us", "GBps", "frac_of_peak", "algorithmic_bytes", "copies")
    out = {}
    g = rotating_gemv(torch, nt, synth.Q8_0, 4096, 4096, 34, 200, 10)
    out["gemv_q8_0_4096x4096"] = {k: g[k] for k in keys}
    torch.cuda.empty_cache()
    lst = []
    for fmt in (synth.Q4_K, synth.Q6_K, synth.Q4_KT):
        for r, c in ((8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672)):
            nbytes = synth.matrix_bytes(fmt, r, c)
            g = rotating_gemv(torch, nt, fmt, r, c, max(2, int(np.ceil(600e6 / nbytes))), 200, 10)
            lst.append({k: g[k] for k in keys})
            log(f"  {g['format']} {r}x{c}: {g['avg_us']:.2f} us, {g['GBps']:.0f} GB/s ({100 * g['frac_of_peak']:.1f}%)")
            torch.cuda.empty_cache()
    out["gemv_70b"] = lst
    out["layer_8b_q8_0"] = layer_8b_measure(torch, nt, tg, 100, 10)
    torch.cuda.empty_cache()
    out["decode_8b_q8_0"] = decode_8b_measure(torch, nt, tg)
    return out


# ----------------------------------------------------------------------------- workloads

def bench_decode_70b(args, torch, nt, tg):
    import synth
    from synth import recipes
    steps = args.steps if args.steps is not None else 128
    warmup = args.warmup if args.warmup is not None else 4
    mix = recipes.MIX_Q4_K_M
    n_layers = args.layers
    log(f"config 4: 70B Q4_K_M, {n_layers} layers resident, {steps} tokens after a 4096-slot cache")
    m = Model70B(torch, nt, tg, mix, n_layers, range(n_layers), tiles=True)
    plan, keep = m.plan()
    head = m.head()
    shp = tg.layer_shape(m.shape)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(m.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    cs = torch.cuda.current_stream().cuda_stream

    def run(n):
        tok.fill_(m.first_token)
        for i in range(n):
            nt.nt_decode_token(None, plan, head, 4096 + i, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                               ws.data_ptr(), wsb, cs, cs, None)

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    tok_s = steps / dt
    last_tok = int(tok.item())
    # the roofline kernel on its own: the fused gate/up launch of every layer back to back
    # (each layer's weights once per round), HIP events around the batch on the launching stream
    fb = ffn_up_bytes(mix, m.shape)
    lw = [m.layer_weights(l) for l in range(n_layers)]
    h_in = torch.from_numpy(recipes.hidden_input(m.shape.dim)).cuda()
    a_out = torch.empty(m.shape.ffn_dim, dtype=torch.float32, device="cuda")

    def ffn(n):
        for i in range(n):
            nt.nt_ffn_up(lw[i % n_layers], shp, h_in.data_ptr(), a_out.data_ptr(), cs)

    ffn(n_layers)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_ffn = 3 * n_layers
    torch.cuda.synchronize()
    ev0.record()
    ffn(n_ffn)
    ev1.record()
    ev1.synchronize()
    ffn_us = ev0.elapsed_time(ev1) * 1e3 / n_ffn
    # per-kernel-class durations inside the decode (separate, instrumented passes over the same
    # tokens; an event pair around every launch adds a few microseconds to each)
    kern = {}
    for name, kc, nbytes in (("ffn_gate_up_swiglu", nt.K_FFN_UP, fb),
                             ("ffn_down_resid", nt.K_FFN_DOWN,
                              synth.matrix_bytes(mix["down"], 8192, 28672) + 4 * (28672 + 2 * 8192)),
                             ("attn_in_qkv_rope", nt.K_ATTN_IN,
                              sum(synth.matrix_bytes(mix[n], *m.shape.matrix_shape(n)) for n in ("q", "k", "v"))
                              + 4 * (2 * 8192 + 8192) + 2 * 2 * 1024),
                             ("attn_o_resid", nt.K_O, synth.matrix_bytes(mix["o"], 8192, 8192) + 4 * 3 * 8192),
                             ("attention", nt.K_ATTN, 2 * 8 * 4160 * 128 * 2 + 4 * 2 * 8192),
                             ("lm_head_argmax", nt.K_LM_HEAD,
                              synth.matrix_bytes(synth.Q4_K, 128256, 8192) + 4 * (2 * 8192 + 128256))):
        kern[name] = timed_class(nt, torch, kc, lambda: run(steps), nbytes)
    tb = np.mean([token_bytes_70b(mix, n_layers, 4096 + i) for i in range(steps)])
    ff = kern["ffn_gate_up_swiglu"]
    res = {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": tok_s, "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": dt / steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (x as three int8 limbs per column with a power-of-two scale per 32 columns), f32 scales, sums and activations, f16 kv (q4_k/q6_k weights)", "data": "synthetic (seeded, random weights of the named shape)",
        "config": {"workload": "llama3.1-70b-shape Q4_K_M resident decode, 128256 vocab, 4096-slot fp16 KV prefill, "
                               "greedy, batch 1 (Q4_K matrices and LM head held in the library's tiled Q4_K layout)", "layers": n_layers, "global_batch": 1, "seq_len": 4096 + steps,
                   "parallelism": "none (1 GPU)"},
        "step_hbm": {"algorithmic_bytes_per_token": int(tb), "GBps": tb * tok_s / 1e9,
                     "frac_of_peak": tb * tok_s / 1e9 / HBM_PEAK_GBS},
        "roofline": {"bound": "hbm", "kernel": "ffn_gate_up_swiglu (fused RMSNorm + Q4_K gate/up GEMV + SwiGLU, tiled Q4_K layout)",
                     "achieved": fb / (ffn_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": fb / (ffn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "bytes_per_launch": fb, "avg_launch_us": ffn_us, "launches": n_ffn,
                     "timing": "HIP events around back-to-back launches over all layers' weights"},
        "kernels": kern,
        "last_token": last_tok,
    }
    # the same step replayed from a HIP graph (one token at a fixed position, captured once)
    # against the same launches enqueued directly: the decode does not need a graph
    res["graph_replay"] = graph_replay(torch, nt, plan, head, m, wsb, ws, h, logits, tok)
    # the yardstick next to the published peak: what plain reads achieve on this part
    rp = read_probe(torch, nt)
    res["read_probe"] = rp
    res["roofline"]["frac_of_read_probe"] = res["roofline"]["achieved"] / rp["GBps"]
    del m, lw, plan, keep
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("GEMV shapes and the 8B layer...")
        res.update(metric_extras(torch, nt, tg))
    if not args.no_cpu_baseline:
        log("cpu baseline (checker on a bounded sample)...")
        res["cpu_baseline"] = cpu_baseline_70b(mix, args.cpu_seconds)
        if not args.no_extras:
            res["cpu_baseline_extras"] = cpu_baseline_extras()
    return res


def graph_replay(torch, nt, plan, head, m, wsb, ws, h, logits, tok, pos=4100, n=32):
    """Per-token time of one decode step (position pos) replayed from a HIP graph, next to the
    same step enqueued directly, and whether the replay reproduces the direct step bit for bit."""
    try:
        s = torch.cuda.Stream()

        def step():
            r = nt.nt_decode_token(None, plan, head, pos, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                                   ws.data_ptr(), wsb, s.cuda_stream, s.cuda_stream, None)
            if r != 0:
                raise RuntimeError(nt.nt_last_error())

        def timed(fn):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) / n * 1e3

        tok.fill_(m.first_token)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            step()
        torch.cuda.synchronize()
        ref = (tok.clone(), h.clone())
        g = torch.cuda.CUDAGraph()
        tok.fill_(m.first_token)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
        torch.cuda.synchronize()
        tok.fill_(m.first_token)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(tok, ref[0]) and torch.equal(h.view(torch.int32), ref[1].view(torch.int32)))
        with torch.cuda.stream(s):
            direct_ms = timed(step)
        replay_ms = timed(g.replay)
        del g
        return {"pos": pos, "tokens": n, "replay_ms_per_token": replay_ms, "direct_ms_per_token": direct_ms,
                "replay_bit_identical": same}
    except Exception as e:  # reported, never fatal to the benchmark line
        return {"error": str(e)}


def rotating_gemv(torch, nt, fmt, rows, cols, copies, steps, warmup, seed=0):
    """Time nt_gemv_q over `copies` distinct weight copies in rotation (past the 256 MB
    last-level cache), HIP events around each launch."""
    import synth
    x = torch.from_numpy(synth.normal_f32(cols, seed, 999)).cuda()
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    nbytes = synth.matrix_bytes(fmt, rows, cols)
    hb = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    cs = torch.cuda.current_stream().cuda_stream
    gen = {synth.Q4_KT: synth.Q4_K, synth.Q8_0T: synth.Q8_0, synth.Q5_KT: synth.Q5_K}.get(fmt, fmt)  # tiled: GGUF blocks rearranged on the device
    ws = []
    for c in range(copies):
        synth.fill_blocks(hb.data_ptr(), gen, nbytes // synth.BLOCK_BYTES[gen], seed, 5000 + c)
        d = hb.cuda()
        if gen != fmt:
            t = torch.empty_like(d)
            nt.nt_repack(fmt, rows, cols, d.data_ptr(), t.data_ptr(), cs)
            d = t
        ws.append(d)

    def run(n):
        for i in range(n):
            nt.nt_gemv_q(fmt, rows, cols, ws[i % copies].data_ptr(), x.data_ptr(), y.data_ptr(), cs)

    run(warmup)
    torch.cuda.synchronize()
    algo = nbytes + 4 * (rows + cols)
    # back to back: HIP events around the whole batch on the launching stream (the kernel's own
    # time, as for the roofline kernel); per launch: an event pair around every launch (adds a few
    # microseconds to each, a large share of the small shapes)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    run(steps)
    ev1.record()
    ev1.synchronize()
    b2b_us = ev0.elapsed_time(ev1) * 1e3 / steps
    r = timed_class(nt, torch, nt.K_GEMV, lambda: run(steps), algo)
    r = {"per_launch_avg_us": r["avg_us"], "per_launch_GBps": r["GBps"], "launches": r["launches"],
         "avg_us": b2b_us, "GBps": algo / (b2b_us * 1e-6) / 1e9}
    r.update({"rows": rows, "cols": cols, "format": synth.FORMAT_NAMES[fmt], "algorithmic_bytes": algo,
              "frac_of_peak": r["GBps"] / HBM_PEAK_GBS, "copies": copies,
              "timing": "avg_us/GBps: HIP events around back-to-back launches; per_launch_*: an event pair per launch"})
    return r


def bench_gemv_shapes(args, torch, nt, tg):
    import synth
    steps = args.steps or 200
    warmup = args.warmup if args.warmup is not None else 10
    out = []
    if args.config == 1:
        shapes = [(synth.Q8_0, 4096, 4096)]
    else:
        shapes = [(f, r, c) for f in (synth.Q4_K, synth.Q6_K, synth.Q5_K, synth.F16, synth.F32, synth.Q4_KT, synth.Q5_KT)
                  for (r, c) in ((8192, 8192), (1024, 8192), (28672, 8192), (8192, 28672))]
    for fmt, r, c in shapes:
        nbytes = synth.matrix_bytes(fmt, r, c)
        copies = max(2, int(np.ceil(600e6 / nbytes)))
        res = rotating_gemv(torch, nt, fmt, r, c, copies, steps, warmup)
        log(f"  {res['format']} {r}x{c}: {res['avg_us']:.2f} us, {res['GBps']:.0f} GB/s ({100 * res['frac_of_peak']:.1f}%) "
            f"back to back; {res['per_launch_avg_us']:.2f} us with an event pair per launch")
        out.append(res)
        torch.cuda.empty_cache()
    best = max(out, key=lambda z: z["algorithmic_bytes"])
    return {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": best["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": best["avg_us"] / 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (x as three int8 limbs per column with a power-of-two scale per 32 columns), f32 scales and sums (quantized weights)", "data": "synthetic",
        "config": {"workload": "Q8_0 GEMV 4096x4096" if args.config == 1 else "70B-shape GEMVs, Q4_K, Q6_K, Q5_K, F16, F32 and tiled Q4_K and Q5_K"},
        "roofline": {"bound": "hbm", "achieved": best["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": best["frac_of_peak"], "traffic": None},
        "gemv": out,
    }


def bench_gemm_tokens(args, torch, nt, tg):
    """The k-token GEMM (nt_gemm_q) at the 70B shapes for k = 1, 2, 4, 8: each weight read
    once per call for all k tokens.  value = weight bytes per second at k = 4 on the
    28672 x 8192 Q4_K shape; every (shape, k) is listed with its GEMV time beside it."""
    import synth
    steps = args.steps or 60
    warmup = args.warmup if args.warmup is not None else 6
    cs = torch.cuda.current_stream().cuda_stream
    out = []
    for fmt, rows, cols in ((synth.Q4_K, 28672, 8192), (synth.Q4_K, 8192, 8192), (synth.Q6_K, 8192, 28672),
                            (synth.Q5_K, 28672, 8192), (synth.Q8_0, 14336, 4096)):
        nbytes = synth.matrix_bytes(fmt, rows, cols)
        copies = max(2, int(np.ceil(600e6 / nbytes)))
        hb = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        ws = []
        for k in range(copies):
            synth.fill_blocks(hb.data_ptr(), fmt, nbytes // synth.BLOCK_BYTES[fmt], 0, 50 + k)
            ws.append(hb.cuda())
        gemv = rotating_gemv(torch, nt, fmt, rows, cols, copies, steps, warmup)
        for k in (1, 2, 4, 8):
            x = torch.from_numpy(np.stack([synth.normal_f32(cols, 0, 60 + t) for t in range(k)])).cuda()
            y = torch.empty(k * rows, dtype=torch.float32, device="cuda")

            def run(n):
                for i in range(n):
                    nt.nt_gemm_q(fmt, rows, cols, k, ws[i % copies].data_ptr(), x.data_ptr(), y.data_ptr(), cs)

            run(warmup)
            torch.cuda.synchronize()
            r = timed_class(nt, torch, nt.K_GEMM, lambda: run(steps), nbytes + 4 * k * (rows + cols))
            # both sides with an event pair per call (a call is one launch per column chunk)
            gv = gemv["per_launch_avg_us"]
            r.update({"format": synth.FORMAT_NAMES[fmt], "rows": rows, "cols": cols, "tokens": k,
                      "gemv_us": gv, "time_vs_gemv": r["avg_us"] / gv,
                      "token_rows_per_us": k * rows / r["avg_us"]})
            log(f"  {r['format']} {rows}x{cols} k={k}: {r['avg_us']:.2f} us ({r['time_vs_gemv']:.2f}x the GEMV's "
                f"{gv:.2f} us), weights at {r['GBps']:.0f} GB/s")
            out.append(r)
        del ws
        torch.cuda.empty_cache()
    head = next(r for r in out if r["format"] == "Q4_K" and r["rows"] == 28672 and r["tokens"] == 4)
    return {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": head["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": head["avg_us"] / 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (x as three int8 limbs per column with a power-of-two scale per 32 columns), f32 scales and sums (quantized weights)", "data": "synthetic",
        "config": {"workload": "k-token quantized GEMM (self-speculative verification), 70B shapes and the 8B Q8_0 FFN shape, k = 1, 2, 4, 8"},
        "roofline": {"bound": "hbm", "achieved": head["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["GBps"] / HBM_PEAK_GBS, "traffic": None},
        "gemm": out,
    }


def bench_layer_skip_70b(args, torch, nt, tg):
    """Cosine-based layer skip on the resident 70B Q4_K_M model: one calibration token runs the
    layers one by one and records cos(h before, h after) per layer (nt_layer_cosine); the
    args.skip layers with the highest similarity are then skipped while decoding.  With random
    weights only the mechanism and its speed are meaningful, not the choice of layers."""
    from synth import recipes
    steps = args.steps if args.steps is not None else 128
    warmup = args.warmup if args.warmup is not None else 4
    mix = recipes.MIX_Q4_K_M
    n_layers = args.layers
    log(f"config 7: 70B Q4_K_M, {n_layers} layers, the {args.skip} most input-like layers skipped")
    m = Model70B(torch, nt, tg, mix, n_layers, range(n_layers), tiles=True)
    head = m.head()
    shp = tg.layer_shape(m.shape)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(m.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    cs = torch.cuda.current_stream().cuda_stream
    # calibration: the first token's embedding row through the layers at pos 4096, one at a time
    tok.fill_(m.first_token)
    nt.nt_embed_row(m.embd_fmt, m.vocab, m.shape.dim, m.embd.data_ptr(), tok.data_ptr(), h.data_ptr(), cs)
    cos = torch.zeros(n_layers, dtype=torch.float32, device="cuda")
    h_in = torch.empty_like(h)
    for l in range(n_layers):
        h_in.copy_(h)
        nt.nt_decode_layer(m.layer_weights(l), shp, 4096, h.data_ptr(), m.kc[l].data_ptr(), m.vc[l].data_ptr(),
                           ws.data_ptr(), wsb, cs)
        nt.nt_layer_cosine(m.shape.dim, h_in.data_ptr(), h.data_ptr(), cos[l:].data_ptr(), cs)
    torch.cuda.synchronize()
    cv = cos.cpu().numpy()
    skip = sorted(int(i) for i in np.argsort(-cv, kind="stable")[:args.skip])
    plan, keep = m.plan(skip=set(skip))
    full, keep_full = m.plan()

    def run(p, n):
        tok.fill_(m.first_token)
        for i in range(n):
            nt.nt_decode_token(None, p, head, 4096 + i, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                               ws.data_ptr(), wsb, cs, cs, None)

    res_t = {}
    for name, p in (("all layers", full), ("skipping", plan)):
        run(p, warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(p, steps)
        torch.cuda.synchronize()
        res_t[name] = steps / (time.perf_counter() - t0)
        log(f"  {name}: {res_t[name]:.2f} tok/s")
    return {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": res_t["skipping"], "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": 1e3 / res_t["skipping"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (x as three int8 limbs per column with a power-of-two scale per 32 columns), f32 scales, sums and activations, f16 kv (q4_k/q6_k weights)", "data": "synthetic (seeded, random weights of the named shape)",
        "config": {"workload": f"llama3.1-70b-shape Q4_K_M resident decode with cosine layer skip ({args.skip} of "
                               f"{n_layers} layers), 4096-slot fp16 KV prefill, greedy, batch 1",
                   "layers": n_layers, "skipped": skip},
        "tok_s_all_layers": res_t["all layers"],
        "layer_cosine": [float(v) for v in cv],
    }


def decode_8b_measure(torch, nt, tg, steps=128, warmup=4):
    """A whole Llama-3-8B-shaped Q8_0 model decoding greedily: 32 layers, Q8_0 embedding and LM
    head (128256 x 4096), 1024-slot caches prefilled with N(0,1) in slots < 1024 - steps, then
    `steps` tokens at positions 1024 - steps .. 1023, host-timed around the loop."""
    from synth import recipes
    import synth
    n0 = recipes.LLAMA3_8B.max_ctx - steps
    m = Model70B(torch, nt, tg, recipes.MIX_Q8_0, 32, range(32), n_prefill=n0, shape=recipes.LLAMA3_8B,
                 head_fmt=synth.Q8_0, tiles=True)
    plan, keep = m.plan()
    head = m.head()
    shp = tg.layer_shape(m.shape)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(m.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    cs = torch.cuda.current_stream().cuda_stream

    def run(pos0, n):
        tok.fill_(m.first_token)
        for i in range(n):
            nt.nt_decode_token(None, plan, head, pos0 + i, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                               ws.data_ptr(), wsb, cs, cs, None)

    run(n0, warmup)  # rewrites slots n0.. that the timed run writes again
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(n0, steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    wbytes = m.lay.nbytes * 32 + synth.matrix_bytes(synth.Q8_0, m.vocab, m.shape.dim)
    kv = 2 * 32 * m.shape.n_kv_heads * m.shape.head_dim * 2 * (n0 + steps / 2)  # average cache read per token
    res = {"tok_s": steps / dt, "ms_per_token": dt / steps * 1e3, "layers": 32, "tokens": steps,
           "positions": [n0, n0 + steps - 1], "weight_bytes_per_token": int(wbytes),
           "GBps": (wbytes + kv) * steps / dt / 1e9, "frac_of_peak": (wbytes + kv) * steps / dt / 1e9 / HBM_PEAK_GBS,
           "last_token": int(tok.item())}
    del m, plan, keep, ws
    torch.cuda.empty_cache()
    return res


def layer_8b_measure(torch, nt, tg, steps, warmup):
    """One Llama-3-8B-shaped Q8_0 decode layer at pos 1023 over a 1024-slot cache, over 4 distinct
    layers' weights in rotation (past the 256 MB last-level cache), host-timed around the batch;
    derived tokens/s = 1 / (32 layers + the Q8_0 128256 x 4096 LM head); the matrices in the
    tiled Q8_0 layout (Q8_0T), as the whole-model measurement holds them."""
    import synth
    from synth import recipes
    shape, mix = recipes.LLAMA3_8B, recipes.MIX_Q8_0
    copies = 4
    lays = [recipes.layer_arrays(shape, mix, l) for l in range(copies)]
    dl = [{k: torch.from_numpy(v).cuda() for k, v in L.items()} for L in lays]
    cs0 = torch.cuda.current_stream().cuda_stream
    for d in dl:
        for n in recipes.TENSORS:
            t = torch.empty_like(d[n])
            nt.nt_repack(synth.Q8_0T, *shape.matrix_shape(n), d[n].data_ptr(), t.data_ptr(), cs0)
            d[n] = t
    ws_list = [tg.layer_weights([synth.Q8_0T] * len(recipes.TENSORS), [d[n] for n in recipes.TENSORS], d["attn_norm"],
                                d["ffn_norm"]) for d in dl]
    kc = torch.from_numpy(recipes.kv_cache_array(shape, 0, "k", 1024)).cuda()
    vc = v_to_device_layout(torch, torch.from_numpy(recipes.kv_cache_array(shape, 0, "v", 1024)).cuda(),
                            shape.n_kv_heads, shape.max_ctx)
    shp = tg.layer_shape(shape)
    wsb = nt.nt_decode_layer_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.from_numpy(recipes.hidden_input(shape.dim)).cuda()
    cs = torch.cuda.current_stream().cuda_stream

    def run(n):
        for i in range(n):
            nt.nt_decode_layer(ws_list[i % copies], shp, 1023, h.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                               ws.data_ptr(), wsb, cs)

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    t_layer = (time.perf_counter() - t0) / steps
    lm = rotating_gemv(torch, nt, synth.Q8_0T, 128256, 4096, 2, 50, 5)
    tok_s = 1.0 / (32 * t_layer + lm["avg_us"] * 1e-6)
    lb = recipes.layer_weight_bytes(shape, mix) + 2 * 8 * 1024 * 128 * 2
    del dl, ws_list
    return {"layer_us": t_layer * 1e6, "layer_GBps": lb / t_layer / 1e9, "layer_frac_of_peak": lb / t_layer / 1e9 / HBM_PEAK_GBS,
            "layer_bytes": lb, "derived_tok_s": tok_s, "roofline_tok_s": 1.0 / ((32 * lb + lm["algorithmic_bytes"]) / (HBM_PEAK_GBS * 1e9)),
            "lm_head_us": lm["avg_us"], "lm_head_GBps": lm["GBps"], "steps": steps}


def bench_layer_8b(args, torch, nt, tg):
    steps = args.steps or 100
    warmup = args.warmup if args.warmup is not None else 10
    r = layer_8b_measure(torch, nt, tg, steps, warmup)
    return {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": r["derived_tok_s"], "unit": "tok/s (derived: 32 layers + Q8_0 LM head)", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": r["layer_us"] / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (x as three int8 limbs per column with a power-of-two scale per 32 columns), f32 scales, sums and activations, f16 kv (q8_0 weights)",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-shape Q8_0 decode layer, pos 1023, 1024-slot fp16 KV"},
        **r,
    }


def bench_stream_70b(args, torch, nt, tg):
    """The 70B Q6_K model with 26 layers resident and 54 streamed from pinned host memory: tokens/s,
    H2D GB/s against a plain pinned copy, and the overlap of copies with compute,
    eta = (T_copy + T_compute - T_total) / min(T_copy, T_compute), from a copy-only pass (the 54 blobs
    copied per token into the two staging buffers, nothing computed) and a compute-only pass (the same
    decode with every layer resident)."""
    from synth import recipes
    steps = args.steps or 32
    warmup = args.warmup if args.warmup is not None else 1
    mix = recipes.MIX_Q6_K
    n_layers = args.layers
    n_res = min(26, n_layers)
    log(f"config 5: 70B Q6_K, {n_res} resident, {n_layers - n_res} streamed from pinned host memory")
    m = Model70B(torch, nt, tg, mix, n_layers, range(n_res))
    plan, keep = m.plan()
    head = m.head()
    shp = tg.layer_shape(m.shape)
    wsb = nt.nt_decode_token_ws_bytes(shp)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    h = torch.zeros(m.shape.dim, dtype=torch.float32, device="cuda")
    logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), m.lay.nbytes)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    stats = nt.StreamStats()
    streamed = sorted(m.host_blobs)
    # plain pinned copy ceiling (one blob at a time, back to back)
    ceil = None
    if streamed:
        probe = m.host_blobs[streamed[0]]
        for _ in range(2):
            with torch.cuda.stream(copy):
                staging[0].copy_(probe, non_blocking=True)
        copy.synchronize()
        t = time.perf_counter()
        for _ in range(3):
            with torch.cuda.stream(copy):
                staging[0].copy_(probe, non_blocking=True)
        copy.synchronize()
        ceil = 3 * m.lay.nbytes / (time.perf_counter() - t) / 1e9

    def run(n, p):
        tok.fill_(m.first_token)
        tot = 0
        for i in range(n):
            nt.nt_decode_token(st, p, head, 4096 + i, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                               ws.data_ptr(), wsb, compute.cuda_stream, copy.cuda_stream, stats)
            tot += stats.h2d_bytes
        return tot

    run(warmup, plan)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    h2d = run(steps, plan)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    t_total = dt / steps
    torch.cuda.synchronize()
    nt.nt_stream_destroy(st)
    # copy-only: the streamed blobs into alternating staging buffers on the copy stream
    n_copy = min(steps, 8)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(copy):
        for i in range(n_copy):
            for j, l in enumerate(streamed):
                staging[j & 1].copy_(m.host_blobs[l], non_blocking=True)
    copy.synchronize()
    t_copy = (time.perf_counter() - t0) / n_copy
    # compute-only: every layer resident (device copies of the streamed blobs)
    dev_copies = {}
    for l in streamed:
        dev_copies[l] = m.host_blobs[l].cuda()
    lay = tg.layer_layout(m.lay.offset_list(), m.lay.fmt_list(), m.lay.nbytes)
    ents = [((m.dev_blobs[l] if l in m.dev_blobs else dev_copies[l]).data_ptr(), True, m.kc[l].data_ptr(),
             m.vc[l].data_ptr()) for l in range(n_layers)]
    rplan, rkeep = tg.model_plan(shp, lay, ents)
    st = None
    run(warmup, rplan)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps, rplan)
    torch.cuda.synchronize()
    t_compute = (time.perf_counter() - t0) / steps
    del dev_copies, rplan, rkeep
    torch.cuda.empty_cache()
    eta = (t_copy + t_compute - t_total) / min(t_copy, t_compute)
    log(f"  total {t_total * 1e3:.1f} ms/token, copy only {t_copy * 1e3:.1f}, compute only {t_compute * 1e3:.1f}, "
        f"eta {eta:.3f}")
    res = {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": steps / dt, "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": dt / steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (x as three int8 limbs per column with a power-of-two scale per 32 columns), "
                 "f32 scales, sums and activations, f16 kv (q6_k weights)",
        "data": "synthetic",
        "config": {"workload": "llama3.1-70b-shape Q6_K, 26 layers resident, 54 streamed from pinned host memory",
                   "layers": n_layers},
        "h2d_GBps": h2d / dt / 1e9, "pinned_copy_ceiling_GBps": ceil, "pcie_gen5_x16_GBps": 63.0,
        "h2d_frac_of_ceiling": (h2d / dt / 1e9) / ceil if ceil else None, "h2d_frac_of_pcie": h2d / dt / 1e9 / 63.0,
        "h2d_bytes_per_token": h2d / steps,
        "overlap": {"t_total_ms": t_total * 1e3, "t_copy_ms": t_copy * 1e3, "t_compute_ms": t_compute * 1e3,
                    "eta": eta, "copy_tokens": n_copy,
                    # the copies are the bound: the streamed token's duration against the copies' alone
                    "copy_rate_vs_alone": t_copy / t_total,
                    "definition": "(T_copy + T_compute - T_total) / min(T_copy, T_compute); T_copy: the streamed "
                                  "blobs copied alone; T_compute: the decode with every layer resident"},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (checker on a bounded sample)...")
        del m
        torch.cuda.empty_cache()
        res["cpu_baseline"] = cpu_baseline_70b(mix, args.cpu_seconds)
    return res


def bench_file_tier_70b(args, torch, nt, tg):
    """The file tier: 70B Q6_K layer blobs written to one file, then decoded with every layer read
    through the page cache into page-locked bounce buffers (args.read_threads pread threads per
    blob), copied to the staging buffers and run; the same layers from pinned host memory beside
    it.  value = file-tier bytes per second (read + H2D, overlapped with compute)."""
    import tempfile
    from synth import recipes
    steps = args.steps or 3
    warmup = args.warmup if args.warmup is not None else 1
    mix = recipes.MIX_Q6_K
    n_layers = args.file_layers
    log(f"config 8: 70B Q6_K, {n_layers} layers read from a file (page cache), {args.read_threads} readers per blob")
    m = Model70B(torch, nt, tg, mix, n_layers, [])
    nb = m.lay.nbytes
    stride = (nb + 4095) // 4096 * 4096
    fdir = os.environ.get("TMPDIR", "/tmp")
    f = tempfile.NamedTemporaryFile(dir=fdir, prefix="nt_layers_", suffix=".bin", delete=False)
    path = f.name
    try:
        for l in range(n_layers):
            f.seek(l * stride)
            f.write(memoryview(m.host_blobs[l].numpy()))
        f.close()
        fd = os.open(path, os.O_RDONLY)
        shp = tg.layer_shape(m.shape)
        lay = tg.layer_layout(m.lay.offset_list(), m.lay.fmt_list(), nb)
        ents = [(0, nt.TIER_FILE, m.kc[l].data_ptr(), m.vc[l].data_ptr(), fd, l * stride) for l in range(n_layers)]
        fplan, keep_f = tg.model_plan(shp, lay, ents)
        pplan, keep_p = m.plan()
        head = m.head()
        wsb = nt.nt_decode_token_ws_bytes(shp)
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        h = torch.zeros(m.shape.dim, dtype=torch.float32, device="cuda")
        logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
        tok = torch.zeros(1, dtype=torch.int32, device="cuda")
        staging = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
        bounce = []
        for _ in range(2):
            t = torch.empty(nb + 4096, dtype=torch.uint8, pin_memory=True)
            off = (-t.data_ptr()) % 4096
            bounce.append(t[off:off + nb])
        st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), nb)
        nt.nt_stream_set_bounce(st, bounce[0].data_ptr(), bounce[1].data_ptr(), nb, args.read_threads)
        compute = torch.cuda.current_stream()
        copy = torch.cuda.Stream()
        stats = nt.StreamStats()
        res = {}
        try:
            for name, plan in (("file", fplan), ("pinned", pplan)):
                def run(n):
                    tok.fill_(m.first_token)
                    tot = 0
                    for i in range(n):
                        nt.nt_decode_token(st, plan, head, 4096 + i, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                                           ws.data_ptr(), wsb, compute.cuda_stream, copy.cuda_stream, stats)
                        tot += stats.h2d_bytes
                    return tot

                run(warmup)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                moved = run(steps)
                torch.cuda.synchronize()
                dt = time.perf_counter() - t0
                res[name] = {"tok_s": steps / dt, "GBps": moved / dt / 1e9, "bytes_per_token": moved / steps}
                log(f"  {name}: {steps / dt:.2f} tok/s, {moved / dt / 1e9:.1f} GB/s of layer blobs")
        finally:
            torch.cuda.synchronize()
            nt.nt_stream_destroy(st)
            os.close(fd)
    finally:
        os.unlink(path)
    return {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": res["file"]["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": 1e3 / res["file"]["tok_s"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (x as three int8 limbs per column with a power-of-two scale per 32 columns), f32 scales, sums and activations, f16 kv (q6_k weights)", "data": "synthetic",
        "config": {"workload": f"llama3.1-70b-shape Q6_K, {n_layers} layers read from a file through the page cache, "
                               f"{args.read_threads} readers per blob", "layers": n_layers},
        "file_tier": res["file"], "pinned_tier": res["pinned"],
    }


def bench_verify_70b(args, torch, nt, tg):
    """The verification pass of self-speculative decoding at the 70B Q4_K_M shape, all layers
    resident: one decode layer for k = 1, 2, 4, 8 tokens at once (nt_decode_layer_k) against
    the single-token layer (nt_decode_layer), each over the 80 layers' weights in turn (HIP
    events around the batch), and the whole-model verify pass (nt_verify_tokens) against k
    single-token steps (nt_decode_token).  value = token positions per second of the k = 4
    verify pass."""
    from synth import recipes
    steps = args.steps if args.steps is not None else 3
    warmup = args.warmup if args.warmup is not None else 1
    mix = recipes.MIX_Q4_K_M
    n_layers = args.layers
    m = Model70B(torch, nt, tg, mix, n_layers, range(n_layers))
    shp = tg.layer_shape(m.shape)
    cs = torch.cuda.current_stream().cuda_stream
    lw = [m.layer_weights(l) for l in range(n_layers)]
    D = m.shape.dim
    pos = 4096
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(run):
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(steps):
            run()
        ev1.record()
        ev1.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / steps

    layers = {}
    ws1 = torch.zeros(nt.nt_decode_layer_ws_bytes(shp), dtype=torch.uint8, device="cuda")
    h1 = torch.from_numpy(recipes.hidden_input(D)).cuda()
    us = timed(lambda: [nt.nt_decode_layer(lw[l], shp, pos, h1.data_ptr(), m.kc[l].data_ptr(), m.vc[l].data_ptr(),
                                           ws1.data_ptr(), ws1.numel(), cs) for l in range(n_layers)])
    t1 = us / n_layers
    layers["single"] = {"us_per_layer": t1}
    for k in (1, 2, 4, 8):
        wsk = torch.zeros(nt.nt_decode_layer_k_ws_bytes(shp, k), dtype=torch.uint8, device="cuda")
        hk = torch.from_numpy(np.tile(recipes.hidden_input(D), k)).cuda()
        us = timed(lambda: [nt.nt_decode_layer_k(lw[l], shp, pos, k, hk.data_ptr(), m.kc[l].data_ptr(),
                                                 m.vc[l].data_ptr(), wsk.data_ptr(), wsk.numel(), cs)
                            for l in range(n_layers)])
        layers[f"k{k}"] = {"us_per_layer": us / n_layers, "vs_k_single_layers": (us / n_layers) / (k * t1)}
        log(f"  layer x{k}: {us / n_layers:.1f} us ({(us / n_layers) / (k * t1):.2f} of {k} single-token layers)")
        del wsk
    plan, keep = m.plan()
    head = m.head()
    passes = {}
    wst = torch.zeros(nt.nt_decode_token_ws_bytes(shp), dtype=torch.uint8, device="cuda")
    h = torch.zeros(D, dtype=torch.float32, device="cuda")
    logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
    tok = torch.full((1,), m.first_token, dtype=torch.int32, device="cuda")
    t_tok = timed(lambda: nt.nt_decode_token(None, plan, head, pos, tok.data_ptr(), logits.data_ptr(), h.data_ptr(),
                                             wst.data_ptr(), wst.numel(), cs, cs, None))
    passes["single_token_step_us"] = t_tok
    for k in (2, 4, 8):
        wsv = torch.zeros(nt.nt_verify_tokens_ws_bytes(shp, k), dtype=torch.uint8, device="cuda")
        hv = torch.zeros(k * D, dtype=torch.float32, device="cuda")
        lv = torch.zeros(k * m.vocab, dtype=torch.float32, device="cuda")
        tin = torch.full((k,), m.first_token, dtype=torch.int32, device="cuda")
        nxt = torch.zeros(k, dtype=torch.int32, device="cuda")
        us = timed(lambda: nt.nt_verify_tokens(None, plan, head, pos, k, tin.data_ptr(), nxt.data_ptr(), lv.data_ptr(),
                                               hv.data_ptr(), wsv.data_ptr(), wsv.numel(), cs, cs, None))
        passes[f"verify_k{k}_us"] = us
        passes[f"verify_k{k}_vs_k_steps"] = us / (k * t_tok)
        log(f"  verify pass x{k}: {us / 1e3:.2f} ms ({us / (k * t_tok):.2f} of {k} single-token steps)")
        del wsv, hv, lv
    v4 = 4 / (passes["verify_k4_us"] * 1e-6)
    return {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": v4, "unit": "token positions/s (k = 4 verify pass)", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": passes["verify_k4_us"] / 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (integer MFMA for Q4_K/Q6_K at k >= 3), f32 scales and activations, f16 kv",
        "data": "synthetic",
        "config": {"workload": "llama3.1-70b-shape Q4_K_M resident, self-speculative verification pass at pos 4096",
                   "layers": n_layers},
        "layers": layers, "passes": passes,
    }


def bench_speculative_stream_70b(args, torch, nt, tg):
    """Self-speculative decoding over the streamed 70B Q6_K model (26 layers resident, 54 streamed
    from pinned host memory): the resident layers draft k - 1 tokens (the streamed ones skipped,
    nothing copied), then the whole model verifies the current token and the drafts in one pass,
    each streamed layer copied once for all k tokens.  value = emitted tokens/s.  With random
    weights the drafts agree with the full model (later layers barely turn the hidden state), so
    the acceptance here measures the mechanism, not a real draft model's quality."""
    from synth import recipes
    k = args.spec_k
    n_out = args.steps if args.steps is not None else 32
    mix = recipes.MIX_Q6_K
    n_layers = args.layers
    n_res = min(26, n_layers)
    m = Model70B(torch, nt, tg, mix, n_layers, range(n_res))
    streamed = set(range(n_res, n_layers))
    full, keep_f = m.plan()
    draft, keep_d = m.plan(skip=streamed)
    head = m.head()
    shp = tg.layer_shape(m.shape)
    D = m.shape.dim
    wst = torch.zeros(nt.nt_decode_token_ws_bytes(shp), dtype=torch.uint8, device="cuda")
    h = torch.zeros(D, dtype=torch.float32, device="cuda")
    logits = torch.zeros(m.vocab, dtype=torch.float32, device="cuda")
    dt = torch.zeros(1, dtype=torch.int32, device="cuda")
    wsv = torch.zeros(nt.nt_verify_tokens_ws_bytes(shp, k), dtype=torch.uint8, device="cuda")
    hv = torch.zeros(k * D, dtype=torch.float32, device="cuda")
    lv = torch.zeros(k * m.vocab, dtype=torch.float32, device="cuda")
    tin = torch.zeros(k, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(k, dtype=torch.int32, device="cuda")
    staging = [torch.empty(m.lay.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    st = nt.nt_stream_create(staging[0].data_ptr(), staging[1].data_ptr(), m.lay.nbytes)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    stats = nt.StreamStats()

    def run(n_emit, pos0):
        out, acc, h2d = [], [], 0
        cur, pos = m.first_token, pos0
        while len(out) < n_emit:
            dt.fill_(cur)
            drafts = []
            for i in range(k - 1):
                nt.nt_decode_token(None, draft, head, pos + i, dt.data_ptr(), logits.data_ptr(), h.data_ptr(),
                                   wst.data_ptr(), wst.numel(), compute.cuda_stream, copy.cuda_stream, None)
                drafts.append(int(dt.item()))
            tin.copy_(torch.tensor([cur] + drafts, dtype=torch.int32))
            nt.nt_verify_tokens(st, full, head, pos, k, tin.data_ptr(), nxt.data_ptr(), lv.data_ptr(), hv.data_ptr(),
                                wsv.data_ptr(), wsv.numel(), compute.cuda_stream, copy.cuda_stream, stats)
            h2d += stats.h2d_bytes
            v = nxt.tolist()
            n = 0
            while n < k - 1 and drafts[n] == v[n]:
                n += 1
            out += v[:n + 1]
            acc.append(n)
            cur, pos = v[n], pos + n + 1
        return out, acc, h2d

    try:
        run(k, 4096)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out, acc, h2d = run(n_out, 4096)
        torch.cuda.synchronize()
        dt_s = time.perf_counter() - t0
    finally:
        torch.cuda.synchronize()
        nt.nt_stream_destroy(st)
    return {
        "metric": "quant-GEMV HBM GB/s (% of peak); decode tokens/s at 8B and 70B shapes",
        "value": len(out) / dt_s, "unit": "tok/s (emitted)", "n_gpus": 1, "steps": len(out), "warmup": k,
        "ms_per_step": dt_s / len(out) * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8 x i8 -> i32 dots (integer MFMA for Q6_K at k >= 3), f32 scales and activations, f16 kv",
        "data": "synthetic (random weights: draft acceptance is an artifact of them)",
        "config": {"workload": f"llama3.1-70b-shape Q6_K, 26 layers resident (the draft model), 54 streamed, "
                               f"self-speculative decoding with k = {k}", "layers": n_layers},
        "verify_passes": len(acc), "accepted_drafts_per_pass": float(np.mean(acc)), "h2d_GBps": h2d / dt_s / 1e9,
        "s_per_pass": dt_s / len(acc),
        "full_acceptance_bound_tok_s": k / (dt_s / len(acc)),  # k tokens per pass if every draft were accepted
        "h2d_bytes_per_emitted_token": h2d / len(out),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this decode path is single-GPU by design "
              "(no sharding or collectives); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_weight_streaming_dequant_amd as nt
    from quantized_weight_streaming_dequant_amd import torch_glue as tg
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(torch)), flush=True)
        return
    nt.load()
    if args.config == 4:
        res = bench_decode_70b(args, torch, nt, tg)
    elif args.config in (1, 3):
        res = bench_gemv_shapes(args, torch, nt, tg)
    elif args.config == 2:
        res = bench_layer_8b(args, torch, nt, tg)
    elif args.config == 6:
        res = bench_gemm_tokens(args, torch, nt, tg)
    elif args.config == 7:
        res = bench_layer_skip_70b(args, torch, nt, tg)
    elif args.config == 8:
        res = bench_file_tier_70b(args, torch, nt, tg)
    elif args.config == 9:
        res = bench_verify_70b(args, torch, nt, tg)
    elif args.config == 10:
        res = bench_speculative_stream_70b(args, torch, nt, tg)
    else:
        res = bench_stream_70b(args, torch, nt, tg)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
