"""MI355X-native quantized-base + low-rank-adapter linear layer (``libqlr.so``).

The library itself is C ABI + gfx950 HIP kernels (``csrc/``, header in
``include/qlr.h``); ``qlr`` is its thin ctypes binding.
"""
from . import qlr
from .qlr import (QWeight, QlrError, codebook, dequantize, force_path, linear, linear_mixed,
                  path, quantize, qweight_sizes, workspace_bytes)

__all__ = ["qlr", "QWeight", "QlrError", "codebook", "dequantize", "force_path", "linear",
           "linear_mixed", "path", "quantize", "qweight_sizes", "workspace_bytes"]
