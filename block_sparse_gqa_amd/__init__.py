"""MiniMax-style block-sparse GQA attention for AMD MI355X (gfx950).

The compute path is libmsa.so (HIP kernels behind the C ABI in include/msa.h); ``msa`` is
its ctypes binding and ``layer`` wires the three calls together on torch-allocated buffers.
"""
from . import msa  # noqa: F401
from .layer import MSALayer  # noqa: F401
