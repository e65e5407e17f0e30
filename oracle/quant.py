"""Blockwise absmax quantization with double quantization.  Test infrastructure.

Follows the QLoRA page: the codebook of section "1. 4-bit NormalFloat (NF4)
quantization" and section "2. Double Quantization", whose arithmetic fixes a
block of 64 weights per first-level constant and an 8-bit second-level code
for each of those constants.

Readings (each one is also listed in the design notes):
  * Block j is the 64 consecutive elements [64j, 64j+64) of the row-major
    flattened weight; its first-level constant is the float32 absmax.  A
    trailing partial block uses the elements present.
  * Code of element w in a block with absmax a: the index of the nearest
    scaled level L[i]*a, ties to the lower index.  Written as a count,
    c = #{i : 2w > (L[i] + L[i+1]) * a}; in float64 both sides are exact
    (L[i] + L[i+1] needs at most 27 significant bits, times a 24-bit a stays
    within 53), so the count equals the exact real-number decision.  a = 0
    gives code 0 everywhere.  Codes are taken from the float32 absmax, before
    that absmax is itself quantized.
  * Packing: block j owns bytes [8bj, 8b(j+1)); element e's code occupies bits
    [b*e, b*e + b) of that little-endian bit string (the page gives only the
    bit count per weight).
  * Double quantization: 256 consecutive first-level constants form a group
    with one float32 constant s = fl32(g/255), g the group's largest absmax;
    each constant gets the 8-bit code of the nearest multiple m*s,
    m in 0..255, ties to the lower m (an unsigned uniform 8-bit grid over
    [0, g]).  The page's "8-bit" says nothing more; one float32 per 256
    blocks is what makes its ~0.127 bits/parameter come out.
  * Dequantization: a' = fl32(code8 * s), w' = fl32(L[c] * a'): exactly two
    float32 multiplies, in that order.  Signed zeros are kept.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .codebook import quantile_codebook

BLOCK = 64
GROUP = 256  # first-level constants per second-level constant


def widen(w: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of the storage dtype to float32 ('bf16' arrays are uint16 bits)."""
    if dtype == "bf16":
        return (np.asarray(w, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype in ("f16", "f32"):
        return np.asarray(w).astype(np.float32)
    raise ValueError(dtype)


def _blocks(flat32: np.ndarray, block: int = BLOCK) -> np.ndarray:
    n = flat32.size
    nblk = -(-n // block)
    padded = np.zeros(nblk * block, dtype=np.float32)
    padded[:n] = flat32
    return padded.reshape(nblk, block)


def block_absmax(flat32: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """float32 max |w| over each block (exact: max of absolute values)."""
    return np.abs(_blocks(flat32, block)).max(axis=1).astype(np.float32)


def nearest_codes(blocks32: np.ndarray, absmax: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Per-element code: count of level midpoints strictly below w (exact fp64)."""
    w2 = 2.0 * blocks32.astype(np.float64)
    a = absmax.astype(np.float64)[:, None]
    lv = levels.astype(np.float64)
    codes = np.zeros(blocks32.shape, dtype=np.int64)
    for i in range(lv.size - 1):
        codes += (w2 > (lv[i] + lv[i + 1]) * a)
    return codes.astype(np.uint8)


def pack_codes(codes: np.ndarray, bits: int, numel: Optional[int] = None) -> np.ndarray:
    """(nblk, 64) codes -> packed bytes, LSB-first per block; absent tail elements -> 0 bits."""
    c = np.array(codes, dtype=np.uint8, copy=True)
    nblk, block = c.shape
    if numel is not None:
        c.reshape(-1)[numel:] = 0
    bitplanes = (c[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1  # (nblk, 64, b)
    return np.packbits(bitplanes.reshape(nblk, block * bits), axis=1, bitorder="little").reshape(-1)


def unpack_codes(packed: np.ndarray, bits: int, nblk: int, block: int = BLOCK) -> np.ndarray:
    """Inverse of pack_codes: packed bytes -> (nblk, 64) codes."""
    by = np.asarray(packed, dtype=np.uint8).reshape(nblk, block * bits // 8)
    bitstr = np.unpackbits(by, axis=1, bitorder="little").reshape(nblk, block, bits)
    weights = (1 << np.arange(bits)).astype(np.uint16)
    return (bitstr.astype(np.uint16) * weights).sum(axis=2).astype(np.uint8)


def double_quantize(absmax: np.ndarray, group: int = GROUP):
    """First-level float32 constants -> (8-bit codes, one float32 step per group).

    s = fl32(g / 255): computed as fl32(fl64(g) / 255); rounding a quotient of
    24-bit operands first to 53 bits and then to 24 gives the same result as
    one rounding, because 53 >= 2*24 + 2.
    """
    nblk = absmax.size
    ngrp = -(-nblk // group)
    padded = np.zeros(ngrp * group, dtype=np.float32)
    padded[:nblk] = absmax
    g = padded.reshape(ngrp, group).max(axis=1)
    step = (g.astype(np.float64) / 255.0).astype(np.float32)
    a = absmax.astype(np.float64)
    s = np.repeat(step.astype(np.float64), group)[:nblk]
    q8 = np.zeros(nblk, dtype=np.int64)
    for m in range(255):
        q8 += (a > (m + 0.5) * s)
    return q8.astype(np.uint8), step


def dequantize_scales(q8: np.ndarray, step: np.ndarray, group: int = GROUP) -> np.ndarray:
    """a'_j = fl32(float(code8_j) * s_group(j))."""
    s = np.repeat(step.astype(np.float32), group)[: q8.size]
    return (q8.astype(np.float32) * s).astype(np.float32)


@dataclasses.dataclass
class QuantizedWeight:
    bits: int
    numel: int
    rows: int
    cols: int
    codes: np.ndarray       # packed uint8
    absmax_q8: np.ndarray   # uint8 per block
    absmax_c: np.ndarray    # float32 per group
    absmax: np.ndarray      # float32 first-level constants (before double quantization)
    code_matrix: np.ndarray  # (nblk, 64) unpacked codes


def quantize(w: np.ndarray, dtype: str, bits: int, rows: Optional[int] = None,
             cols: Optional[int] = None) -> QuantizedWeight:
    """Quantize a weight array of any shape (flattened row-major)."""
    flat = widen(w, dtype).reshape(-1)
    if not np.all(np.isfinite(flat)):
        raise ValueError("non-finite weight")
    levels = quantile_codebook(bits)
    blocks = _blocks(flat)
    absmax = np.abs(blocks).max(axis=1).astype(np.float32)
    codes = nearest_codes(blocks, absmax, levels)
    codes.reshape(-1)[flat.size:] = 0
    q8, step = double_quantize(absmax)
    if rows is None:
        rows, cols = (w.shape if w.ndim == 2 else (1, flat.size))
    return QuantizedWeight(bits, flat.size, rows, cols, pack_codes(codes, bits, flat.size), q8,
                           step, absmax, codes)


def dequantize(codes_packed: np.ndarray, q8: np.ndarray, step: np.ndarray, bits: int,
               numel: int) -> np.ndarray:
    """float32 w'_e = fl32(L[c_e] * a'_j), flattened, first ``numel`` elements."""
    levels = quantile_codebook(bits)
    nblk = q8.size
    c = unpack_codes(codes_packed, bits, nblk)
    a_deq = dequantize_scales(q8, step)
    w = (levels[c.astype(np.int64)] * a_deq[:, None]).astype(np.float32)
    return w.reshape(-1)[:numel]


def qweight_sizes(rows: int, cols: int, bits: int):
    """(codes bytes, absmax_q8 bytes, absmax_c bytes) for a rows x cols weight."""
    numel = rows * cols
    nblk = -(-numel // BLOCK)
    ngrp = -(-nblk // GROUP)
    return nblk * BLOCK * bits // 8, nblk, 4 * ngrp
