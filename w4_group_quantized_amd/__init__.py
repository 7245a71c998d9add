"""MI355X (gfx950) sparse-MoE expert layer with int4 g128 experts.

The compute path is libmoe_w4.so (hand-written HIP kernels behind a C ABI,
include/moe_w4.h); this package is its thin Python binding.  Importing it
fails if the library has not been built: there is no fallback.
"""
from . import _native  # noqa: F401  (raises ImportError when libmoe_w4.so is missing)
from ._native import MoeError, MOE_RMSNORM  # noqa: F401
from .layer import (W4MoELayer, W4MoEStack, MoEBuffers, quantize_fp16, quantize_w8,  # noqa: F401
                    dequantize, pack_plain)
