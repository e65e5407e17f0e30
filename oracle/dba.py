"""Double-binary adapter branch (LoRDBA) on the quantized base.  Test infrastructure.

LoRDBA page (gist.science summary), section 2 "Core architecture": the adapter
update is a sum over an envelope rank l of diag(alpha_i) B1 diag(beta_i) B2
diag(gamma_i), with sign factors B1 (N x R) and B2 (R x K) in {-1, +1} (one bit
per entry) shared by the l terms, and per-channel scale vectors alpha_i (N),
beta_i (R), gamma_i (K) stored in fp16.  In adapter mode the update stays a
separate branch beside the frozen base (sections 1-2):

    y = x W'^T + x dW^T,   x dW^T = sum_i alpha_i * (((x * gamma_i) B2^T) * beta_i) B1^T

with * the per-channel (broadcast) product: the page's two sign-accumulate
products interleaved with channel scales.

Readings (the page prints no format): a sign bit 1 stands for +1 and 0 for -1;
B1 row n is R bits and B2 row j is K bits, each packed LSB-first into 32-bit
words (row stride ceil(R/32) and ceil(K/32) words); alpha, beta, gamma are
fp16 arrays of shape (l, N), (l, R), (l, K).  All arithmetic here is float64
on exactly widened values.
"""
from __future__ import annotations

import numpy as np

from .quant import widen


def pack_signs(S: np.ndarray) -> np.ndarray:
    """(rows, cols) array of +-1 -> uint32 (rows, ceil(cols/32)), bit c % 32 of word c // 32 is 1 for +1."""
    S = np.asarray(S)
    if S.ndim != 2 or not np.all(np.abs(S) == 1):
        raise ValueError("signs must be a matrix of +-1")
    rows, cols = S.shape
    words = (cols + 31) // 32
    out = np.zeros((rows, words), dtype=np.uint64)
    for c in range(cols):
        out[:, c // 32] |= (S[:, c] > 0).astype(np.uint64) << np.uint64(c % 32)
    return out.astype(np.uint32)


def unpack_signs(P: np.ndarray, cols: int) -> np.ndarray:
    """Inverse of pack_signs: uint32 (rows, words) -> float64 (rows, cols) of +-1."""
    P = np.asarray(P, dtype=np.uint32)
    bits = np.array([(P[:, c // 32] >> np.uint32(c % 32)) & np.uint32(1) for c in range(cols)]).T
    return np.where(bits == 1, 1.0, -1.0)


def delta_w(alpha, beta, gamma, b1_packed, b2_packed):
    """dW = sum_i diag(alpha_i) B1 diag(beta_i) B2 diag(gamma_i) (N x K, float64).

    alpha (l, N), beta (l, R), gamma (l, K) as fp16 arrays (or float arrays of
    fp16 values); b1_packed (N, ceil(R/32)), b2_packed (R, ceil(K/32)) uint32.
    """
    al, be, ga = (np.asarray(v, dtype=np.float64) for v in (alpha, beta, gamma))
    if al.ndim != 2 or be.ndim != 2 or ga.ndim != 2 or not (al.shape[0] == be.shape[0] == ga.shape[0]):
        raise ValueError("alpha, beta, gamma must be (l, N), (l, R), (l, K)")
    N, R, K = al.shape[1], be.shape[1], ga.shape[1]
    B1 = unpack_signs(b1_packed, R)
    B2 = unpack_signs(b2_packed, K)
    if B1.shape != (N, R) or B2.shape != (R, K):
        raise ValueError("sign factors do not match the scale vectors")
    dW = np.zeros((N, K))
    for i in range(al.shape[0]):
        dW += (al[i][:, None] * B1 * be[i][None, :]) @ (B2 * ga[i][None, :])
    return dW


def linear_dba(x, xdtype, wdeq32, alpha, beta, gamma, b1_packed, b2_packed):
    """y = x W'^T + x dW^T (adapter mode), float64, following the page's two
    sign-accumulate stages with the channel scales between them."""
    xf = widen(x, xdtype).astype(np.float64)
    w = wdeq32.astype(np.float64)
    if xf.ndim != 2 or xf.shape[1] != w.shape[1]:
        raise ValueError("x must be (M, K) and W' (N, K)")
    al, be, ga = (np.asarray(v, dtype=np.float64) for v in (alpha, beta, gamma))
    R, K = be.shape[1], ga.shape[1]
    B1 = unpack_signs(b1_packed, R)
    B2 = unpack_signs(b2_packed, K)
    y = xf @ w.T
    for i in range(al.shape[0]):
        z = (xf * ga[i][None, :]) @ B2.T          # stage 1: M x R, sums of +-x*gamma
        y = y + ((z * be[i][None, :]) @ B1.T) * al[i][None, :]   # stage 2, then alpha
    return y


def linear_dba_tolerance(x, xdtype, wdeq32, alpha, beta, gamma, b1_packed, b2_packed):
    """S[m, n] = sum_k |x w'| + sum_i |alpha_i[n]| sum_j |beta_i[j]| sum_k |x[m,k] gamma_i[k]|."""
    xf = np.abs(widen(x, xdtype).astype(np.float64))
    S = xf @ np.abs(wdeq32.astype(np.float64)).T
    al, be, ga = (np.abs(np.asarray(v, dtype=np.float64)) for v in (alpha, beta, gamma))
    for i in range(al.shape[0]):
        z = xf @ ga[i]                            # M, sum_k |x gamma|
        S = S + np.outer(z * be[i].sum(), al[i])
    return S


def adapter_bits(N, K, R, l):
    """Stored bits of the adapter: sign factors N R + R K, fp16 scales 16 l (N + R + K)."""
    return N * R + R * K + 16 * l * (N + R + K)
