"""Pins of the oracle's forward y = x W'^T + s (x A^T) B^T (unmerged adapter branch)."""
import math

import numpy as np
import pytest

import oracle
import workloads


def _small(seed=0, M=3, N=5, K=128, r=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = (rng.standard_normal((r, K)) / math.sqrt(K)).astype(np.float32)
    B = (rng.standard_normal((N, r)) * 0.01).astype(np.float32)
    return x, w, A, B


def test_fsum_brute_force():
    x, w, A, B = _small()
    s = 0.75
    y = oracle.linear(x, "f32", w, A, B, "f32", s)
    M, K = x.shape
    N, r = B.shape
    for m in range(M):
        t = [math.fsum(float(x[m, k]) * float(A[j, k]) for k in range(K)) for j in range(r)]
        for n in range(N):
            base = math.fsum(float(x[m, k]) * float(w[n, k]) for k in range(K))
            lora = math.fsum(t[j] * float(B[n, j]) for j in range(r))
            ref = base + s * lora
            assert abs(y[m, n] - ref) <= 1e-12 * (abs(ref) + 1e-3)


def test_rank_zero_and_zero_B_give_the_base():
    x, w, A, B = _small(1)
    base = oracle.linear(x, "f32", w)
    assert np.array_equal(oracle.linear(x, "f32", w, A, np.zeros_like(B), "f32", 2.0), base)
    assert np.array_equal(oracle.linear(x, "f32", w, A[:0], B[:, :0], "f32", 2.0), base)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.allclose(base, ref, rtol=0, atol=1e-14)


def test_merged_equals_unmerged():
    """Adapter mode (unmerged) and merged weights give the same product up to fp64 rounding."""
    x, w, A, B = _small(2, M=4, N=7, K=192, r=3)
    s = 1.5
    y = oracle.linear(x, "f32", w, A, B, "f32", s)
    merged = w.astype(np.float64) + s * (B.astype(np.float64) @ A.astype(np.float64))
    y2 = x.astype(np.float64) @ merged.T
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-14)


def test_linear_in_x():
    x, w, A, B = _small(3)
    y1 = oracle.linear(x, "f32", w, A, B, "f32", 0.5)
    assert np.allclose(oracle.linear(2 * x, "f32", w, A, B, "f32", 0.5), 2 * y1, rtol=1e-13, atol=1e-15)
    # superposition with disjoint supports (so x1 + x2 == x exactly in float32)
    x1, x2 = x.copy(), x.copy()
    x1[:, 64:] = 0
    x2[:, :64] = 0
    ya = oracle.linear(x1, "f32", w, A, B, "f32", 0.5)
    yb = oracle.linear(x2, "f32", w, A, B, "f32", 0.5)
    assert np.allclose(ya + yb, y1, rtol=1e-12, atol=1e-15)


def test_operand_orientation_is_enforced():
    x, w, A, B = _small(5, M=2, N=6, K=128, r=3)
    with pytest.raises(ValueError):
        oracle.linear(x, "f32", w, A.T.copy(), B, "f32", 1.0)
    with pytest.raises(ValueError):
        oracle.linear(x, "f32", w, A, B.T.copy(), "f32", 1.0)


def test_tolerance_scale():
    x, w, _, _ = _small(6)
    S = oracle.linear_tolerance(x, "f32", w)
    for m in range(x.shape[0]):
        for n in range(w.shape[0]):
            ref = math.fsum(abs(float(x[m, k]) * float(w[n, k])) for k in range(x.shape[1]))
            assert abs(S[m, n] - ref) <= 1e-12 * ref
    assert np.all(S >= np.abs(oracle.linear(x, "f32", w)) * (1 - 1e-12))


def test_bf16_inputs_widen_exactly():
    lin = workloads.make_linear("t", 99, 8, 64, 2, sigma=0.02, wdtype="f32", bits=4, r=2,
                                alpha=4.0, abdtype="bf16", xdtype="bf16")
    xf = oracle.widen(lin.x, "bf16").astype(np.float64)
    Af = oracle.widen(lin.A, "bf16").astype(np.float64)
    assert np.allclose(oracle.lora_t(lin.x, "bf16", lin.A, "bf16"), xf @ Af.T, rtol=0, atol=0)


def test_end_to_end_tiny_workload():
    lin = workloads.tiny()
    qw = oracle.quantize(lin.W, "f32", 4)
    wd = oracle.dequantize(qw.codes, qw.absmax_q8, qw.absmax_c, 4, lin.W.size).reshape(lin.W.shape)
    y = oracle.linear(lin.x, "f32", wd, lin.A, lin.B, "f32", lin.scale)
    assert y.shape == (8, 256) and np.all(np.isfinite(y))
    # quantization error of the base product is small against its scale
    yq = oracle.linear(lin.x, "f32", lin.W.astype(np.float32))
    S = oracle.linear_tolerance(lin.x, "f32", wd)
    assert np.max(np.abs(oracle.linear(lin.x, "f32", wd) - yq) / S) < 0.2
