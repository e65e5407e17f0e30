"""CPU oracle for the quantized-base + low-rank-adapter linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  The GPU library never calls it and shares no code, table or constant
with it.

Plain, slow, obviously correct numpy: every floating-point decision is taken in
float64 on exactly representable operands (so it is exact), and every rounding
to float32 is an explicit, single IEEE rounding.  Each function cites the page
passage it follows; where the pages leave a step open the reading taken is
stated beside it.

Pages (titles as printed):
  * "QLoRA" (aizip.shop methodologies page): the k-bit NormalFloat codebook
    equation, the double-quantization paragraph with its bits/parameter
    arithmetic, and the memory-decomposition equation.
  * "LoRDBA" (gist.science summary): the unmerged "adapter mode", in which the
    frozen quantized base and the adapter branch stay separate terms.
  * "AutoQRA" (gist.science summary), section 3.1: one (bits, rank) pair per
    layer (a mixed stack is a list of independent ``quantize`` + ``linear``
    entries, each with its own bits and rank); section 1: the quantized backbone is frozen and adapters are trained
    (the backward in ``linear``).
  * "LoRDBA" section 2: the double-binary adapter branch (``dba``).
  * "QFT" (gist.science summary), section 2.2: the hybrid outlier split
    (``outliers``).
  * "QWHA" (gist.science summary), section 2.1: the Walsh-Hadamard adapter
    (``wha``).

Every function here is pinned by a ``-m "not gpu"`` test against something
other than itself (closed forms, brute force over exact rationals, invariants,
page arithmetic); no function is "parity unpinned".
"""
from .codebook import normal_quantile, quantile_codebook
from .quant import (widen, block_absmax, nearest_codes, pack_codes, unpack_codes,
                    double_quantize, dequantize_scales, dequantize, quantize,
                    qweight_sizes, QuantizedWeight)
from .linear import (lora_t, linear, linear_tolerance, linear_backward,
                     linear_backward_tolerance, adapter_grads, adapter_grads_tolerance)
from . import dba, outliers, wha

__all__ = [
    "normal_quantile", "quantile_codebook", "widen", "block_absmax", "nearest_codes",
    "pack_codes", "unpack_codes", "double_quantize", "dequantize_scales", "dequantize",
    "quantize", "qweight_sizes", "QuantizedWeight", "lora_t", "linear",
    "linear_tolerance", "linear_backward", "linear_backward_tolerance", "adapter_grads",
    "adapter_grads_tolerance", "dba", "outliers", "wha",
]
