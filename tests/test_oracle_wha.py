"""Pins of the oracle's Walsh-Hadamard adapter (QWHA page, section 2.1)."""
import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads
from oracle import outliers as oo
from oracle import wha


@pytest.mark.parametrize("P", [1, 2, 4, 8, 16, 64, 256])
def test_hadamard_is_the_textbook_matrix(P):
    """Natural (Sylvester) order, as scipy builds it; only +-1 entries; H H = P I; symmetric."""
    H = wha.hadamard(P)
    assert np.array_equal(H, scipy.linalg.hadamard(P).astype(np.float64))
    assert np.all(np.abs(H) == 1)
    assert np.array_equal(H @ H, P * np.eye(P)) and np.array_equal(H, H.T)


def _fast_wht(v):
    """The textbook recursion H_2n = [[H_n, H_n], [H_n, -H_n]] as in-place butterflies
    (additions and subtractions only), on a copy of the vector."""
    v = np.array(v, dtype=np.float64)
    h = 1
    while h < v.size:
        for i in range(0, v.size, 2 * h):
            a, b = v[i:i + h].copy(), v[i + h:i + 2 * h].copy()
            v[i:i + h], v[i + h:i + 2 * h] = a + b, a - b
        h *= 2
    return v


@pytest.mark.parametrize("K,P", [(64, 64), (64, 16), (96, 32), (256, 256)])
def test_rows_transform_equals_butterflies_and_inverse(K, P):
    rng = np.random.default_rng(K + P)
    x = rng.integers(-5, 6, size=(3, K)).astype(np.float32)
    z = wha.wht_rows(x, "f32", P)
    for m in range(3):
        ref = np.concatenate([_fast_wht(x[m, b * P:(b + 1) * P]) for b in range(K // P)]) / P
        assert np.array_equal(z[m], ref)
    # H^-1 = H / P: the transform matrix over P is its own inverse
    T = wha.transform_matrix(K, P)
    assert np.allclose(np.linalg.inv(T), T / P, rtol=0, atol=1e-12)
    # energy: ||x H||^2 = P ||x||^2, so ||z||^2 = ||x||^2 / P
    assert np.allclose((z ** 2).sum(axis=1), (x.astype(np.float64) ** 2).sum(axis=1) / P, rtol=1e-13)


def test_bad_blocks_are_rejected():
    for K, P in [(64, 3), (64, 128), (96, 64), (64, 0)]:
        with pytest.raises(ValueError):
            wha.transform_matrix(K, P)


@pytest.mark.parametrize("K,P", [(64, 64), (128, 32)])
def test_single_coefficient_is_a_square_wave(K, P):
    """F with one entry c at (n, j): dW row n is c/P times row j of H inside j's block, zero elsewhere."""
    N, n, j, c = 5, 3, 37, 2.5
    csr = (np.array([0, 0, 0, 0, 1, 1], dtype=np.int32), np.array([j], dtype=np.int32),
           np.array([c], dtype=np.float32))
    dW = wha.delta_w(csr, N, K, P)
    assert not np.delete(dW, n, axis=0).any()
    b = j // P
    Hp = wha.hadamard(P)
    expect = np.zeros(K)
    expect[b * P:(b + 1) * P] = c * Hp[j % P] / P
    assert np.array_equal(dW[n], expect)
    assert set(np.abs(dW[n][b * P:(b + 1) * P])) == {c / P}


@pytest.mark.parametrize("P", [16, 64])
def test_merged_equals_unmerged_exactly(P):
    """Small-integer x, W' and c: every product is exact in float64 (P a power of two)."""
    rng = np.random.default_rng(P)
    M, N, K = 4, 6, 64
    x = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    w = rng.integers(-4, 5, size=(N, K)).astype(np.float32)
    row_ptr, col, val = workloads.wha_coefficients(N, K, 20, cfg=3, floor=2)
    val = np.round(val * 4).astype(np.float32)
    csr = (row_ptr, col, val)
    y = wha.linear_wht(x, "f32", w, csr, P)
    merged = x.astype(np.float64) @ (w.astype(np.float64) + wha.delta_w(csr, N, K, P)).T
    assert np.array_equal(y, merged)
    # F = 0 gives the base; an F with the outlier-channel format and x replaced by z is the same sparse product
    zero = (row_ptr, col, np.zeros_like(val))
    assert np.array_equal(wha.linear_wht(x, "f32", w, zero, P), oracle.linear(x, "f32", w))
    z = wha.wht_rows(x, "f32", P)
    assert np.array_equal(y - oracle.linear(x, "f32", w), z @ oo.sparse_dense(csr, N, K).T)


def test_tolerance_bounds_and_single_term_equality():
    rng = np.random.default_rng(9)
    M, N, K, P = 3, 5, 128, 32
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    csr = workloads.wha_coefficients(N, K, 30, cfg=4, floor=1)
    y = wha.linear_wht(x, "f32", w, csr, P)
    S = wha.linear_wht_tolerance(x, "f32", w, csr, P)
    assert np.all(np.abs(y) <= S * (1 + 1e-12))
    # one coefficient, a zero base, x >= 0 on its block and j = block start (row j of H is all +1):
    # the term equals its magnitude sum exactly
    xp = np.abs(x)
    one = (np.array([0, 1, 1, 1, 1, 1], dtype=np.int32), np.array([64], dtype=np.int32),
           np.array([1.5], dtype=np.float32))
    y1 = wha.linear_wht(xp, "f32", np.zeros_like(w), one, P)
    S1 = wha.linear_wht_tolerance(xp, "f32", np.zeros_like(w), one, P)
    assert np.allclose(y1[:, 0], S1[:, 0], rtol=1e-13, atol=0)


def test_coefficient_generator_budget_floor_and_rows():
    N, K = 64, 256
    row_ptr, col, val = workloads.wha_coefficients(N, K, 2048, cfg=5, floor=16)
    counts = np.diff(row_ptr)
    assert row_ptr[0] == 0 and row_ptr[-1] == 2048 and counts.min() >= 16 and counts.max() <= K
    assert counts.max() > counts.min()  # uneven allocation
    for n in range(N):
        seg = col[row_ptr[n]:row_ptr[n + 1]]
        assert np.all(np.diff(seg) > 0) and seg.min() >= 0 and seg.max() < K


def test_rows_transform_per_block_equals_the_block_diagonal_matrix():
    """wht_rows forms each block separately; the full block-diagonal product gives the same values."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 192)).astype(np.float32)
    for P in (1, 8, 64):
        z = wha.wht_rows(x, "f32", P)
        ref = x.astype(np.float64) @ wha.transform_matrix(192, P) / P
        assert np.allclose(z, ref, rtol=1e-14, atol=1e-15)
