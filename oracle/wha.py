"""Walsh-Hadamard adapter (QWHA) on the quantized base.  Test infrastructure.

QWHA page (gist.science summary), section 2.1 "Adapter design: Walsh-Hadamard
adaptation": the weight update is a single transform, dW = F H^-1, with H the
Walsh-Hadamard matrix (entries +-1 only) and F a sparse trainable coefficient
matrix given by a value vector c and an index list E.  In adapter mode the
update stays a separate branch beside the frozen base:

    y = x W'^T + x dW^T,   x dW^T = (x H^-T) F^T.

Readings (the page gives no size rule, ordering, format or scaling):
  * H is the natural-order (Sylvester) Hadamard matrix, H[i][j] =
    (-1)^popcount(i & j), so H is symmetric, H H = P I and H^-1 = H / P.
  * The transform acts on the input dimension in blocks of P = a power of two
    dividing K (H = blockdiag of K / P copies of H_P); P = K is the single full
    transform.  Shapes such as K = 11008 = 2^8 * 43 need blocks.
  * F is N x K, stored as CSR by output row (row_ptr, col = transform index,
    val = c in float32), the same format as the outlier side channel.
  * Hence x dW^T = z F^T with z = x blockdiag(H_P) / P: a fast transform of each
    x row (additions and subtractions only, as the page stresses) and one
    exact power-of-two scaling, then a sparse product.
All arithmetic here is float64 on exactly widened values.
"""
from __future__ import annotations

import numpy as np

from .quant import widen
from .outliers import sparse_dense


def _check_block(K: int, P: int) -> None:
    if P < 1 or P & (P - 1) or K % P:
        raise ValueError("P must be a power of two dividing K")


def hadamard(P: int) -> np.ndarray:
    """The P x P natural-order Walsh-Hadamard matrix, H[i][j] = (-1)^popcount(i & j), float64."""
    _check_block(P, P)
    i = np.arange(P, dtype=np.int64)
    a = i[:, None] & i[None, :]
    parity = np.zeros_like(a)
    while np.any(a):
        parity ^= a & 1
        a >>= 1
    return np.where(parity == 1, -1.0, 1.0)


def transform_matrix(K: int, P: int) -> np.ndarray:
    """blockdiag(H_P, ..., H_P), K x K float64."""
    _check_block(K, P)
    H = np.zeros((K, K))
    Hp = hadamard(P)
    for b in range(K // P):
        H[b * P:(b + 1) * P, b * P:(b + 1) * P] = Hp
    return H


def wht_rows(x, xdtype: str, P: int) -> np.ndarray:
    """z = x blockdiag(H_P) / P (float64), i.e. x H^-T with H^-1 = H / P.

    Written per block (block b of z is block b of x times H_P): the same product
    as with the full block-diagonal matrix, without forming it for wide K."""
    x64 = widen(x, xdtype).astype(np.float64)
    M, K = x64.shape
    _check_block(K, P)
    Hp = hadamard(P)
    z = np.empty_like(x64)
    for b in range(K // P):
        z[:, b * P:(b + 1) * P] = x64[:, b * P:(b + 1) * P] @ Hp
    return z / P


def delta_w(csr, N: int, K: int, P: int) -> np.ndarray:
    """The dense update dW = F H^-1 (N x K, float64)."""
    return sparse_dense(csr, N, K) @ (transform_matrix(K, P) / P)


def linear_wht(x, xdtype: str, wdeq32, csr, P: int) -> np.ndarray:
    """y = x W'^T + (x H^-T) F^T, float64."""
    from .linear import linear
    N, K = wdeq32.shape
    return linear(x, xdtype, wdeq32) + wht_rows(x, xdtype, P) @ sparse_dense(csr, N, K).T


def linear_wht_tolerance(x, xdtype: str, wdeq32, csr, P: int) -> np.ndarray:
    """S[m, n] = sum_k |x w'| + sum_j |c_j| (sum over block(j) of |x_k|) / P: the magnitude sum of
    every product that defines y[m, n] (each z_j is a signed sum of the |x_k| of its block over P)."""
    xa = np.abs(widen(x, xdtype).astype(np.float64))
    N, K = wdeq32.shape
    _check_block(K, P)
    blk = xa.reshape(xa.shape[0], K // P, P).sum(axis=2) / P          # (M, K/P)
    zmag = np.repeat(blk, P, axis=1)                                   # (M, K): |z_j| bound per j
    return xa @ np.abs(wdeq32.astype(np.float64)).T + zmag @ np.abs(sparse_dense(csr, N, K)).T
