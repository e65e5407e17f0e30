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


def linear_backward(dy, dydtype, x, xdtype, wdeq32, A=None, B=None, abdtype="f32", scale=0.0):
    """Gradients of the forward above for an upstream gradient dy (M x N), float64.

    The pages freeze the quantized base and train only the adapter (QLoRA page,
    memory-decomposition equation: frozen 4-bit weights, bf16 adapters with
    optimizer state; AutoQRA page, "1. Problem statement": the quantized backbone
    stays frozen while lightweight adapters are trained).  The gradients are not
    written out on the pages; they are the chain rule of the forward, the plain
    definition used here:
        u  = dy B                    (M x r)
        t  = x A^T                   (M x r)
        dx = dy W' + scale u A       (M x K)   input gradient through the frozen base
        dA = scale u^T x             (r x K)
        dB = scale dy^T t            (N x r)
    W' itself gets no gradient.  Returns (dx, dA, dB); dA and dB are None when
    the call has no adapter.
    """
    g = _f64(dy, dydtype)
    xf = _f64(x, xdtype)
    w = wdeq32.astype(np.float64)
    if g.ndim != 2 or xf.ndim != 2 or w.ndim != 2:
        raise ValueError("dy, x and W' must be matrices")
    if xf.shape[1] != w.shape[1] or g.shape != (xf.shape[0], w.shape[0]):
        raise ValueError("x must be (M, K), W' (N, K) and dy (M, N)")
    dx = g @ w
    if A is None or B is None or A.shape[0] == 0:
        return dx, None, None
    Af, Bf = _f64(A, abdtype), _f64(B, abdtype)
    if Af.shape[1] != w.shape[1] or Bf.shape != (w.shape[0], Af.shape[0]):
        raise ValueError("A must be (r, K) and B (N, r)")
    dx = dx + float(scale) * ((g @ Bf) @ Af)
    dA, dB = adapter_grads(dy, dydtype, x, xdtype, A, B, abdtype, scale)
    return dx, dA, dB


def adapter_grads(dy, dydtype, x, xdtype, A, B, abdtype, scale):
    """The adapter's gradients alone (they do not involve W'), float64:
    dA = scale (dy B)^T x  (r x K),  dB = scale dy^T (x A^T)  (N x r)."""
    g, xf = _f64(dy, dydtype), _f64(x, xdtype)
    Af, Bf = _f64(A, abdtype), _f64(B, abdtype)
    if Af.shape[1] != xf.shape[1] or Bf.shape != (g.shape[1], Af.shape[0]) or g.shape[0] != xf.shape[0]:
        raise ValueError("dy (M, N), x (M, K), A (r, K) and B (N, r) do not fit together")
    s = float(scale)
    u = g @ Bf
    t = xf @ Af.T
    return s * (u.T @ xf), s * (g.T @ t)


def linear_backward_tolerance(dy, dydtype, x, xdtype, wdeq32, A=None, B=None, abdtype="f32", scale=0.0):
    """Magnitude sums that scale the per-element error bound of each gradient.

    Every term of each gradient is replaced by its absolute value, and so is every
    term of the intermediate u = dy B and t = x A^T that feeds it (their rounding
    errors are bounded by the same sums):
        Sdx[m,k] = sum_n |dy w'| + |s| sum_j U[m,j] |A[j,k]|,  U = |dy| |B|
        SdA[j,k] = |s| sum_m U[m,j] |x[m,k]|
        SdB[n,j] = |s| sum_m |dy[m,n]| T[m,j],                 T = |x| |A|^T
    """
    g = np.abs(_f64(dy, dydtype))
    xf = np.abs(_f64(x, xdtype))
    w = np.abs(wdeq32.astype(np.float64))
    sdx = g @ w
    if A is None or B is None or A.shape[0] == 0:
        return sdx, None, None
    Af, Bf = np.abs(_f64(A, abdtype)), np.abs(_f64(B, abdtype))
    sdx = sdx + abs(float(scale)) * ((g @ Bf) @ Af)
    sdA, sdB = adapter_grads_tolerance(dy, dydtype, x, xdtype, A, B, abdtype, scale)
    return sdx, sdA, sdB


def adapter_grads_tolerance(dy, dydtype, x, xdtype, A, B, abdtype, scale):
    """SdA and SdB of linear_backward_tolerance alone."""
    g, xf = np.abs(_f64(dy, dydtype)), np.abs(_f64(x, xdtype))
    Af, Bf = np.abs(_f64(A, abdtype)), np.abs(_f64(B, abdtype))
    s = abs(float(scale))
    U = g @ Bf
    T = xf @ Af.T
    return s * (U.T @ xf), s * (g.T @ T)
