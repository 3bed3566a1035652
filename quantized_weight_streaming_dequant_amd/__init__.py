"""nt: batch-1 decode over block-quantized weights on AMD Instinct MI355X (gfx950).

The compute path is libnt.so (hand-written HIP kernels behind the C ABI in
include/nt.h); this package only binds it.  Importing the package does not load
the library; the first call does, and raises if it is missing.
"""
from ._abi import *  # noqa: F401,F403
from ._abi import (EXPORTS, LIB_PATH, LayerEntry, LayerLayout, LayerShape, LayerWeights, ModelHead, ModelPlan,
                   NtError, StreamStats, load, last_error, version)

__all__ = [n for n in dir() if not n.startswith("_")]
