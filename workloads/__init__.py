"""Seeded synthetic inputs for the quantized-base + low-rank-adapter linear layer.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
no arithmetic of the method itself: it only draws random numbers and rounds
them to the storage dtypes (fp16 by numpy's IEEE cast, bf16 by round-to-nearest-
even from fp32).  bf16 arrays are returned as ``uint16`` bit patterns because
numpy has no bf16 type.

Recipe (every tensor): ``numpy.random.default_rng(SeedSequence([seed, cfg,
tensor_id, *extra]))`` (PCG64), standard normals drawn in float32 and scaled by
the stated sigma in float32, then cast to the storage dtype.

The shapes follow the layer sizes the pages talk about (a 7B-class model's
attention and MLP projections, and a 65B-class MLP projection: QLoRA page,
section on the memory decomposition and the 65B example); the pretrained
weights are replaced by N(0, sigma^2) draws, which is the distribution the
QLoRA page gives as the premise of the NormalFloat codebook.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# tensor ids inside one config
T_W, T_A, T_B, T_X, T_OUTLIER, T_DRAW, T_DY = 0, 1, 2, 3, 4, 5, 6

BITS_CHOICES = (2, 3, 4, 8)
RANK_CHOICES = (4, 8, 16, 32, 64)


def rng_for(cfg: int, *ids: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, *ids]))


def normal(shape, sigma: float, cfg: int, *ids: int, seed: int = 0) -> np.ndarray:
    g = rng_for(cfg, *ids, seed=seed)
    z = g.standard_normal(size=shape, dtype=np.float32)
    return z * np.float32(sigma)


def to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "f16":
        return a32.astype(np.float16)
    if dtype == "bf16":
        return to_bf16_bits(a32)
    raise ValueError(dtype)


@dataclasses.dataclass
class Linear:
    """One linear layer's synthetic inputs (all host numpy arrays).

    W: (N, K) in ``wdtype``; A: (r, K); B: (N, r) in ``abdtype``;
    x: (M, K) in ``xdtype``; scale = alpha / r.
    """
    name: str
    W: np.ndarray
    wdtype: str
    bits: int
    r: int
    alpha: float
    A: Optional[np.ndarray]
    B: Optional[np.ndarray]
    abdtype: str
    x: np.ndarray
    xdtype: str
    cfg: int = 0
    sub: int = 0

    @property
    def N(self) -> int:
        return self.W.shape[0]

    @property
    def K(self) -> int:
        return self.W.shape[1]

    @property
    def M(self) -> int:
        return self.x.shape[0]

    @property
    def scale(self) -> float:
        return float(np.float32(self.alpha) / np.float32(self.r)) if self.r > 0 else 0.0


def make_weight(cfg: int, N: int, K: int, sigma: float, wdtype: str, sub: int = 0,
                outlier_frac: float = 0.0, outlier_mult: float = 20.0, seed: int = 0) -> np.ndarray:
    w = normal((N, K), sigma, cfg, T_W, sub, seed=seed)
    if outlier_frac > 0.0:
        cnt = int(round(outlier_frac * N * K))
        pos = rng_for(cfg, T_OUTLIER, sub, seed=seed).choice(N * K, size=cnt, replace=False)
        flat = w.reshape(-1)
        flat[pos] = flat[pos] * np.float32(outlier_mult)
    return store(w, wdtype)


def make_linear(name: str, cfg: int, N: int, K: int, M: int, *, sigma: float, wdtype: str,
                bits: int, r: int, alpha: float, abdtype: str, xdtype: str,
                a_sigma: Optional[float] = None, b_sigma: float = 0.01, sub: int = 0,
                outlier_frac: float = 0.0, seed: int = 0, W: Optional[np.ndarray] = None) -> Linear:
    if W is None:
        W = make_weight(cfg, N, K, sigma, wdtype, sub=sub, outlier_frac=outlier_frac, seed=seed)
    if a_sigma is None:
        a_sigma = float(np.sqrt(1.0 / K))
    A = store(normal((r, K), a_sigma, cfg, T_A, sub, seed=seed), abdtype) if r > 0 else None
    B = store(normal((N, r), b_sigma, cfg, T_B, sub, seed=seed), abdtype) if r > 0 else None
    x = store(normal((M, K), 1.0, cfg, T_X, sub, M, seed=seed), xdtype)
    return Linear(name, W, wdtype, bits, r, alpha, A, B, abdtype, x, xdtype, cfg, sub)


T_DBA = 7


@dataclasses.dataclass
class DbaAdapter:
    """A double-binary adapter's synthetic storage: random sign words and fp16 scales.

    b1 (N, ceil(R/32)) and b2 (R, ceil(K/32)) uint32 words of independent fair
    bits (padding bits random too: the format ignores them); alpha (l, N),
    beta (l, R), gamma (l, K) fp16 draws of N(0, 0.01^2), N(0, 1) and N(0, 1/K),
    so that one term of the update has the scale of a LoRA update with
    B ~ N(0, 0.01^2) and A ~ N(0, 1/K).
    """
    R: int
    ell: int
    b1: np.ndarray
    b2: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    gamma: np.ndarray


def dba_adapter(N: int, K: int, R: int, ell: int, cfg: int = 0, sub: int = 0, seed: int = 0) -> DbaAdapter:
    g = rng_for(cfg, T_DBA, sub, R, ell, seed=seed)
    b1 = g.integers(0, 2 ** 32, size=(N, (R + 31) // 32), dtype=np.uint64).astype(np.uint32)
    b2 = g.integers(0, 2 ** 32, size=(R, (K + 31) // 32), dtype=np.uint64).astype(np.uint32)
    alpha = (g.standard_normal((ell, N), dtype=np.float32) * np.float32(0.01)).astype(np.float16)
    beta = g.standard_normal((ell, R), dtype=np.float32).astype(np.float16)
    gamma = (g.standard_normal((ell, K), dtype=np.float32) * np.float32(np.sqrt(1.0 / K))).astype(np.float16)
    return DbaAdapter(R, ell, b1, b2, alpha, beta, gamma)


T_WHA = 8


def wha_coefficients(N: int, K: int, budget: int, cfg: int = 0, sub: int = 0, seed: int = 0,
                     floor: int = 0, sigma: float = 0.5):
    """A sparse coefficient matrix F (N x K) in CSR form (row_ptr int32, col int32, val float32).

    ``budget`` coefficients in all, at least ``floor`` per row; the rest spread
    over the rows in proportion to a lognormal per-row weight, so that some
    rows get many more than others (the shape of an error-proportional
    allocation).  Positions within a row are distinct, uniform, ascending;
    values N(0, sigma^2).  The default sigma gives a 32-coefficient row at
    P = 4096 the entry scale of a rank-16 LoRA update with B ~ N(0, 0.01^2),
    A ~ N(0, 1/K).
    """
    g = rng_for(cfg, T_WHA, sub, budget, seed=seed)
    if not N * floor <= budget <= N * K:
        raise ValueError("budget out of range")
    wgt = np.exp(g.standard_normal(N))
    counts = np.full(N, floor, dtype=np.int64)
    extra = g.multinomial(budget - N * floor, wgt / wgt.sum())
    counts += extra
    # cap at K and hand the excess to rows with room, in row order
    over = np.maximum(counts - K, 0).sum()
    counts = np.minimum(counts, K)
    for n in range(N):
        if over == 0:
            break
        add = min(K - counts[n], over)
        counts[n] += add
        over -= add
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col = np.empty(budget, dtype=np.int32)
    for n in range(N):
        col[row_ptr[n]:row_ptr[n + 1]] = np.sort(g.choice(K, size=int(counts[n]), replace=False))
    val = (g.standard_normal(budget, dtype=np.float32) * np.float32(sigma)).astype(np.float32)
    return row_ptr.astype(np.int32), col, val


def upstream_grad(lin: Linear, seed: int = 0) -> np.ndarray:
    """A synthetic upstream gradient dy (M x N) for the backward, N(0, 1) in x's dtype.

    The pages give no gradient statistics; a standard normal of the output's
    shape is the plain stand-in (the same draw as x, on the other side).
    """
    return store(normal((lin.M, lin.N), 1.0, lin.cfg, T_DY, lin.sub, lin.M, seed=seed), lin.xdtype)


# ---------------------------------------------------------------- the five workloads

def tiny(seed: int = 0) -> Linear:
    """256x256 fp32 weights, 4-bit, rank 4 (alpha 8) fp32 adapters, 8x256 fp32 x."""
    return make_linear("tiny", 1, 256, 256, 8, sigma=0.02, wdtype="f32", bits=4, r=4,
                       alpha=8.0, abdtype="f32", xdtype="f32", a_sigma=float(np.sqrt(1 / 256)),
                       seed=seed)


def attn(M: int, seed: int = 0, W: Optional[np.ndarray] = None) -> Linear:
    """7B-class attention projection 4096x4096 fp16 with 0.1% x20 outliers, 4-bit, r16 a16."""
    return make_linear(f"attn_M{M}", 2, 4096, 4096, M, sigma=0.02, wdtype="f16", bits=4, r=16,
                       alpha=16.0, abdtype="bf16", xdtype="bf16", outlier_frac=0.001,
                       seed=seed, W=W)


def mlp(which: str, M: int, seed: int = 0, W: Optional[np.ndarray] = None) -> Linear:
    """7B-class MLP projection: 'up' 11008x4096 or 'down' 4096x11008, fp16, 4-bit, r64 a16."""
    N, K, sub = (11008, 4096, 0) if which == "up" else (4096, 11008, 1)
    return make_linear(f"mlp_{which}_M{M}", 3, N, K, M, sigma=0.02, wdtype="f16", bits=4, r=64,
                       alpha=16.0, abdtype="bf16", xdtype="bf16", sub=sub, seed=seed, W=W)


def big65(M: int, seed: int = 0, W: Optional[np.ndarray] = None) -> Linear:
    """65B-class MLP projection 22016x8192 fp16 (sigma 0.015), 4-bit, r64 a16."""
    return make_linear(f"big65_M{M}", 5, 22016, 8192, M, sigma=0.015, wdtype="f16", bits=4,
                       r=64, alpha=16.0, abdtype="bf16", xdtype="bf16", seed=seed, W=W)


MIXED_SHAPES: Tuple[Tuple[int, int], ...] = ((4096, 4096),) * 4 + ((11008, 4096),) * 2 + ((4096, 11008),)
MIXED_LAYERS = 32


def mixed_plan(seed: int = 0, layers: int = MIXED_LAYERS) -> List[Tuple[int, int, int, int]]:
    """(N, K, bits, rank) for every linear of the mixed stack, layer-major."""
    g = rng_for(4, T_DRAW, seed=seed)
    n = layers * len(MIXED_SHAPES)
    bits = g.choice(np.array(BITS_CHOICES), size=n)
    ranks = g.choice(np.array(RANK_CHOICES), size=n)
    plan = []
    for i in range(n):
        N, K = MIXED_SHAPES[i % len(MIXED_SHAPES)]
        plan.append((N, K, int(bits[i]), int(ranks[i])))
    return plan


def mixed_linear(i: int, M: int = 512, seed: int = 0, plan=None,
                 shape_override: Optional[Tuple[int, int]] = None) -> Linear:
    """Linear number ``i`` of the mixed stack (independent of the others).

    ``shape_override`` keeps the drawn (bits, rank) but shrinks (N, K); tests use
    it to run the stack at sizes the oracle finishes quickly.
    """
    plan = plan or mixed_plan(seed)
    N, K, bits, r = plan[i]
    if shape_override is not None:
        N, K = shape_override
    return make_linear(f"mixed_{i}", 4, N, K, M, sigma=0.02, wdtype="f16", bits=bits, r=r,
                       alpha=16.0, abdtype="bf16", xdtype="bf16", sub=1000 + i, seed=seed)


# ---------------------------------------------------------------- inputs drawn on the GPU

def device_normal(shape, sigma: float, dtype, device, cfg: int, *ids: int, seed: int = 0):
    """N(0, sigma^2) drawn on the GPU by torch's seeded generator, in float32, scaled by sigma in
    float32 and cast to ``dtype`` (a torch dtype).  For inputs too large to draw on the host in
    reasonable time (the full mixed stack): the seed is a function of (seed, cfg, *ids) only, so a
    draw is reproducible; it is a different sample than ``normal`` draws for the same ids."""
    import torch
    state = np.random.SeedSequence([seed, cfg, *ids]).generate_state(2, dtype=np.uint32)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(state[0]) << 32 | int(state[1]))
    z = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return (z * np.float32(sigma)).to(dtype)


def device_mixed_linear(i: int, M: int, device, plan=None, seed: int = 0):
    """Linear number ``i`` of the mixed stack with its inputs drawn on the GPU (``device_normal``):
    returns (N, K, bits, r, alpha, W fp16, x bf16, A bf16, B bf16) with the distributions of
    ``mixed_linear`` (W N(0, 0.02^2), A N(0, 1/K), B N(0, 0.01^2), x N(0, 1), alpha 16)."""
    import torch
    plan = plan or mixed_plan(seed)
    N, K, bits, r = plan[i]
    sub = 1000 + i
    W = device_normal((N, K), 0.02, torch.float16, device, 4, T_W, sub, seed=seed)
    x = device_normal((M, K), 1.0, torch.bfloat16, device, 4, T_X, sub, M, seed=seed)
    A = device_normal((r, K), float(np.sqrt(1.0 / K)), torch.bfloat16, device, 4, T_A, sub, seed=seed)
    B = device_normal((N, r), 0.01, torch.bfloat16, device, 4, T_B, sub, seed=seed)
    return N, K, bits, r, 16.0, W, x, A, B
