"""Helpers for the GPU parity tests: device buffers, streams and tolerance checks."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def zeros_u8(n: int) -> torch.Tensor:
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_rel(got, ref, nrm, tol=1e-3, what=""):
    """|got - ref| <= tol * nrm elementwise; where nrm == 0, got must be exactly 0."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nrm = np.asarray(nrm, dtype=np.float64)
    assert got.shape == ref.shape == nrm.shape, (got.shape, ref.shape, nrm.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    zero = nrm == 0
    assert np.all(got[zero] == 0), f"{what}: nonzero output where the normaliser is 0"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, nrm))
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= tol, f"{what}: worst relative error {ratio[worst]:.3e} at {worst} (got {got.flat[worst]}, ref {ref.flat[worst]})"
    return float(ratio.max())


def same_value(a, b) -> bool:
    """Bit-exact comparison by value (so -0 == +0), NaN-free inputs."""
    a = np.asarray(a)
    b = np.asarray(b)
    return a.shape == b.shape and bool(np.all(a == b))


def v_to_device(vc, n_kv: int, max_ctx: int, hd: int = 128) -> np.ndarray:
    """[n_kv][max_ctx][hd] V cache -> the library's layout [n_kv][max_ctx/8][hd][8]
    (groups of 8 slots, slot-minor)."""
    a = np.asarray(vc).reshape(n_kv, max_ctx // 8, 8, hd)
    return np.ascontiguousarray(a.transpose(0, 1, 3, 2))


def v_from_device(vt, n_kv: int, max_ctx: int, hd: int = 128) -> np.ndarray:
    """Inverse of v_to_device."""
    a = np.asarray(vt).reshape(n_kv, max_ctx // 8, hd, 8)
    return np.ascontiguousarray(a.transpose(0, 1, 3, 2)).reshape(n_kv, max_ctx, hd)


def check_layer_stages(st: dict, g: dict, what: str = "") -> dict:
    """Judge one decode layer stage by stage against the checker's teacher-forced run st
    (oracle.decode_layer with forced = the GPU's k16, v16, q, o, h1, a): the fp16 cache entries
    within the GEMV tolerance of the exact value plus half a binary16 step; the rotated query,
    the attention output, h1, the SwiGLU output and h2 within 1e-3 of their normalisers.
    g holds the GPU's k16, v16 (bits), q, o, h1, a and h2.  Returns the worst ratio per stage."""
    # RoPE mixes rows 2i and 2i+1: the pair's GEMV normalisers bound the rotated error
    qn = np.repeat(st["q_nrm"][0::2] + st["q_nrm"][1::2], 2)
    kn = np.repeat(st["k_nrm"][0::2] + st["k_nrm"][1::2], 2)
    res = {}
    for name, exact, nrm in (("k16", st["k"], kn), ("v16", st["v"], st["v_nrm"])):
        bits = np.asarray(g[name], dtype=np.uint16)
        val = bits.view(np.float16).astype(np.float64)
        half_step = np.spacing(np.abs(bits.view(np.float16))).astype(np.float64) / 2
        err = np.abs(val - exact)
        assert np.all(err <= 1e-3 * nrm + half_step), \
            f"{what} {name}: worst {np.max(err / (1e-3 * nrm + half_step)):.3f}"
        res[name] = float(np.max(np.maximum(err - half_step, 0) / nrm))
    res["q"] = check_rel(g["q"], st["q"], qn, what=f"{what} q")
    res["o"] = check_rel(g["o"], st["o"], st["o_nrm"], what=f"{what} attention")
    res["h1"] = check_rel(g["h1"], st["h1"], st["h1_nrm"], what=f"{what} h1")
    # a = silu(g) u: with |dg| <= e N_g and |du| <= e N_u, |da| <= e (1.1 N_g |u| + |g| N_u) + O(e^2)
    na = 1.1 * st["gate_nrm"] * np.abs(st["up"]) + (np.abs(st["gate"]) + 1e-3 * st["gate_nrm"]) * st["up_nrm"]
    res["a"] = check_rel(g["a"], st["a"], na, what=f"{what} swiglu")
    res["h2"] = check_rel(g["h2"], st["h2"], st["h2_nrm"], what=f"{what} h2")
    return res
