"""MI355X (gfx950) forward pass of one DeepSeekMoE-style MoE FFN layer.

The work runs in hand-written HIP kernels behind the C ABI of ``libmoe.so``
(``include/moe.h``).  This package holds the kernels' sources (``csrc/``), the
build script and a thin ctypes binding; PyTorch only supplies device memory
and streams.  There is no fallback path: if the library is missing, loading
fails.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    MOE_BF16,
    MOE_F32,
    PATH_AUTO,
    PATH_DECODE,
    PATH_PREFILL,
    Diag,
    Dims,
    Library,
    MoeError,
    Options,
    Weights,
    load,
)
from .layer import MoELayer, capacity_seats  # noqa: F401
