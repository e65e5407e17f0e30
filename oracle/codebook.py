"""k-bit quantile ("NormalFloat") codebook.  Test infrastructure (see package header).

QLoRA page, section "1. 4-bit NormalFloat (NF4) quantization": level i is the
standard-normal quantile function Q_N evaluated at probability (i - 1/2)/2^b,
b = 4 giving 16 levels.

Readings (the page leaves these open or prints them garbled):
  * The printed index range i = 0..2^b-1 together with (i - 1/2) would put
    probability < 0 at i = 0, so the index is read as 1-based; with a 0-based
    i the probability is (i + 1/2)/2^b.
  * The levels are divided by the largest quantile Q_N((2^b - 1/2)/2^b) so that
    they span [-1, 1] (absmax scaling maps each block onto [-1, 1]).
  * The lower half is computed and the upper half is its mirror image,
    L[n-1-i] = -L[i]; with an even count there is no exact zero level.
  * Each level is rounded once, to nearest-even float32, from a 50-digit value.
"""
from __future__ import annotations

import functools

import mpmath
import numpy as np

_DPS = 50


def normal_quantile(p) -> mpmath.mpf:
    """Q_N(p) = sqrt(2) * erfinv(2p - 1), at 50 significant digits."""
    with mpmath.workdps(_DPS):
        p = mpmath.mpf(p)
        return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)


def _round_f32(v: mpmath.mpf) -> float:
    """Round a high-precision value to float32 (nearest, ties even) in one step."""
    with mpmath.workprec(24):
        r = +v  # unary plus rounds to the working precision
    out = float(r)  # exact: r has 24 significant bits
    assert float(np.float32(out)) == out
    return out


def quantile_codebook(bits: int) -> np.ndarray:
    """The 2^bits ascending float32 levels L[0..2^bits-1] (readings above)."""
    return _codebook(bits).copy()


@functools.lru_cache(maxsize=None)
def _codebook(bits: int) -> np.ndarray:
    if bits < 1 or bits > 8:
        raise ValueError("bits must be in 1..8")
    n = 1 << bits
    with mpmath.workdps(_DPS):
        top = normal_quantile(mpmath.mpf(2 * n - 1) / (2 * n))
        lower = []
        for i in range(n // 2):
            z = normal_quantile(mpmath.mpf(2 * i + 1) / (2 * n))
            lower.append(_round_f32(z / top))
    levels = lower + [-v for v in reversed(lower)]
    return np.array(levels, dtype=np.float32)
