"""Hybrid outlier split of the frozen weight (QFT).  Test infrastructure.

QFT page (gist.science summary), section 2.2 "Hybrid feature quantizer": a
small fraction of the weights (about 1 %), the outliers that stretch the
dynamic range, are kept at full precision in a sparse part; the dense rest is
quantized.  Here the dense rest uses this library's quantized format (the
QLoRA page's blockwise quantile codes with double-quantized scales) in place of
QFT's uniform INT8, and the forward adds the sparse part as a separate term:

    y = x W'^T + x S^T (+ the adapter branch),

W' the dequantized dense part and S the sparse outliers (float32 values).

Readings (the page gives no rule): the outliers are the k entries with the
largest |w| (float32 after exact widening), ties broken by the lower flat
(row-major) index; their positions are 0 in the dense part before it is
quantized.  The quantile codebook has no exact zero level, so a zeroed entry
still dequantizes to a small nonzero w'; the sparse value is therefore the
residual val = fl32(w - w') (one rounding), which makes W' + S return w at the
outlier positions up to that rounding.  S is stored as CSR by weight row
(row_ptr int32[rows + 1], col int32[k], val float32[k]), columns ascending
within a row.  k is the caller's count (the attention workload's
round(0.1 % N K) planted outliers).
"""
from __future__ import annotations

import numpy as np

from .quant import widen, quantize, dequantize


def select_outliers(w32_flat: np.ndarray, k: int) -> np.ndarray:
    """Flat indices of the k largest |w|, ties to the lower index; returned ascending."""
    w = np.asarray(w32_flat, dtype=np.float32).reshape(-1)
    if not 0 <= k <= w.size:
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(w.size), -np.abs(w.astype(np.float64))))  # |w| descending, then index
    return np.sort(order[:k])


def split(w, dtype: str, rows: int, cols: int, k: int):
    """(dense float32 flat array with the outliers zeroed, their flat indices, the widened w)."""
    w32 = widen(np.asarray(w).reshape(-1), dtype).astype(np.float32)
    if w32.size != rows * cols:
        raise ValueError("w must hold rows * cols elements")
    idx = select_outliers(w32, k)
    dense = w32.copy()
    dense[idx] = 0.0
    return dense, idx, w32


def csr_of(idx, vals, rows: int, cols: int):
    """CSR (row_ptr, col, val) of entries at ascending flat indices idx."""
    r, c = idx // cols, idx % cols
    row_ptr = np.zeros(rows + 1, dtype=np.int64)
    np.add.at(row_ptr, r + 1, 1)
    return np.cumsum(row_ptr).astype(np.int32), c.astype(np.int32), np.asarray(vals, dtype=np.float32)


def quantize_with_outliers(w, dtype: str, bits: int, rows: int, cols: int, k: int):
    """(QuantizedWeight of the dense part, CSR of the residuals at the outliers)."""
    dense, idx, w32 = split(w, dtype, rows, cols, k)
    q = quantize(dense, "f32", bits)
    deq = dequantize(q.codes, q.absmax_q8, q.absmax_c, bits, dense.size)
    vals = (w32[idx].astype(np.float64) - deq[idx].astype(np.float64)).astype(np.float32)
    return q, csr_of(idx, vals, rows, cols)


def sparse_dense(csr, rows: int, cols: int) -> np.ndarray:
    """S as a dense float64 rows x cols matrix."""
    row_ptr, col, val = csr
    S = np.zeros((rows, cols))
    for n in range(rows):
        for j in range(int(row_ptr[n]), int(row_ptr[n + 1])):
            S[n, int(col[j])] += float(val[j])
    return S


def linear_outliers(x, xdtype, wdeq32, csr, A=None, B=None, abdtype="f32", scale=0.0):
    """y = x W'^T + x S^T + scale (x A^T) B^T, float64."""
    from .linear import linear
    y = linear(x, xdtype, wdeq32, A, B, abdtype, scale)
    S = sparse_dense(csr, wdeq32.shape[0], wdeq32.shape[1])
    return y + widen(x, xdtype).astype(np.float64) @ S.T


def linear_outliers_tolerance(x, xdtype, wdeq32, csr):
    """S_tol[m, n] = sum_k |x w'| + sum_j |x[m, col_j] val_j| (the base scale plus the sparse terms)."""
    xa = np.abs(widen(x, xdtype).astype(np.float64))
    S = np.abs(sparse_dense(csr, wdeq32.shape[0], wdeq32.shape[1]))
    return xa @ np.abs(wdeq32.astype(np.float64)).T + xa @ S.T
