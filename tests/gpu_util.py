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
