"""Build libnt.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libnt.so")

SOURCES = ["gemv.hip", "attn.hip", "small.hip", "layer_k.hip", "abi.cpp", "noalloc.cpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, out: str = LIB, defines: tuple = (), build_dir: str = BUILD) -> str:
    """Compile every source and link libnt.so at `out` (defines: extra -D flags)."""
    os.makedirs(build_dir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        dflags = [f"-D{d}" for d in defines]
        cmd = [HIPCC, *FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC, *[f for f in FLAGS if f != "--offload-arch=gfx950"], *dflags, "-x", "hip",
                   "--offload-arch=gfx950", "-c", os.path.join(CSRC, src), "-o", obj]
        objs.append(obj)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = False
    for src, p in procs:
        log, _ = p.communicate()
        log = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l and "ignoring feature" not in l)
        if p.returncode != 0:
            failed = True
            print(f"--- hipcc failed on {src}:\n{log}", file=sys.stderr)
        elif verbose and log.strip():
            print(log, file=sys.stderr)
    if failed:
        raise RuntimeError("HIP build failed")
    tmp = out + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
