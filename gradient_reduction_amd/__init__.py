"""MI355X-native data-parallel gradient reduction: DeepCompile-style ZeRO-1
bucket flush (AllReduce / reduce-to-owner), reduce-scatter / all-gather slab
layouts and deferred reduction under gradient accumulation, over W simulated
ranks held as rows of one GPU's [W, M] gradient slab.

The computation lives in libdc.so (hand-written HIP for gfx950, C ABI in
include/dc.h); `dc` binds it, `executor` drives a bucket sequence and
`deferred` the accumulate-then-reduce sequence of a gradient-accumulation
step.
"""
from . import dc  # noqa: F401
from .dc import DCError  # noqa: F401

__all__ = ["dc", "DCError"]
