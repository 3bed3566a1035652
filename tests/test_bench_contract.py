"""The benchmark's output contract: one JSON line with the fields the harness reads, and a
refusal of more than one GPU.  The GPU case runs a 2-layer model in a child process."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    """--gpus 2 exits with status 2 and says why, before it touches a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.gpu
def test_bench_line_has_every_field():
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--layers", "2", "--steps", "3",
                        "--warmup", "1", "--cpu-seconds", "1"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert "workload" in d["config"]
    rf = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in rf, k
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    cb = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cb, k
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
    assert cb["one_thread"]["cores"] == 1 and cb["one_thread"]["value"] > 0
    ce = d["cpu_baseline_extras"]
    assert ce["kind"] == "oracle" and ce["one_thread"]["cores"] == 1
    assert ce["all"]["gemv_q8_0_4096x4096"]["GBps"] > 0 and ce["all"]["layer_8b_q8_0"]["seconds"] > 0
    # the GEMV and 8B halves of the metric ride along in the default line
    assert d["gemv_q8_0_4096x4096"]["GBps"] > 0 and len(d["gemv_70b"]) == 12
    assert d["layer_8b_q8_0"]["derived_tok_s"] > 0
    assert d["decode_8b_q8_0"]["tok_s"] > 0 and d["decode_8b_q8_0"]["layers"] == 32
    # the step replayed from a HIP graph reproduces the direct step
    gr = d["graph_replay"]
    assert "error" not in gr, gr
    assert gr["replay_bit_identical"] and gr["replay_ms_per_token"] > 0
