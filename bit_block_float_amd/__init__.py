"""HiFloat4 (HiF4) W4A4 fake-quantized linear layers on MI355X (gfx950).

The product is libhif4.so (C ABI: include/hif4.h) over hand-written HIP
kernels; ``bit_block_float_amd.hif4`` is its thin Python binding.
"""
from . import hif4  # noqa: F401

__all__ = ["hif4"]
