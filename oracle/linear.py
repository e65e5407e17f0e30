"""Forward of the frozen quantized base plus an unmerged low-rank adapter.  Test infrastructure.

y = x W'^T + s (x A^T) B^T, with W' the dequantized base (N x K), A (r x K),
B (N x r), s = alpha / r.  The pages keep the base frozen in 4 bits and the
adapters in bf16 (QLoRA page, memory-decomposition equation and the remark
after it) and serve the adapter unmerged as a separate branch (LoRDBA page,
section 1 and the "adapter mode" protocol of section 2).  The low-rank product
and its alpha/r scale are the standard LoRA form the QLoRA page names as a
prerequisite; they are not written out on the pages.

All products and sums are float64 (numpy matmul on widened, exact inputs).
"""
from __future__ import annotations

import numpy as np

from .quant import widen


def _f64(a, dtype):
    return widen(a, dtype).astype(np.float64)


def lora_t(x, xdtype, A, abdtype):
    """t = x A^T (M x r), float64."""
    return _f64(x, xdtype) @ _f64(A, abdtype).T


def linear(x, xdtype, wdeq32, A=None, B=None, abdtype="f32", scale=0.0):
    """y = x W'^T + scale (x A^T) B^T in float64.  ``wdeq32``: (N, K) float32."""
    xf = _f64(x, xdtype)
    w = wdeq32.astype(np.float64)
    if xf.ndim != 2 or w.ndim != 2 or xf.shape[1] != w.shape[1]:
        raise ValueError("x must be (M, K) and W' (N, K)")
    y = xf @ w.T
    if A is not None and B is not None and A.shape[0] > 0:
        Af, Bf = _f64(A, abdtype), _f64(B, abdtype)
        if Af.shape[1] != w.shape[1] or Bf.shape != (w.shape[0], Af.shape[0]):
            raise ValueError("A must be (r, K) and B (N, r)")
        t = xf @ Af.T
        y = y + float(scale) * (t @ Bf.T)
    return y


def linear_tolerance(x, xdtype, wdeq32):
    """S[m, n] = sum_k |x[m,k] * w'[n,k]|: the scale of the per-element error bound."""
    return np.abs(_f64(x, xdtype)) @ np.abs(wdeq32.astype(np.float64)).T


def mixed(entries):
    """Independent linears: ``entries`` is a list of kwargs for ``linear``."""
    return [linear(**e) for e in entries]
