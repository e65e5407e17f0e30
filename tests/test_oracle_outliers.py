"""Pins of the oracle's hybrid outlier split (QFT page, section 2.2)."""
import numpy as np
import pytest

import oracle
import workloads
from oracle import outliers as oo


def _brute_select(w, k):
    keyed = sorted(range(len(w)), key=lambda i: (-abs(float(w[i])), i))
    return sorted(keyed[:k])


@pytest.mark.parametrize("seed,n,k", [(0, 50, 5), (1, 64, 0), (2, 64, 64), (3, 200, 17)])
def test_selection_brute_force(seed, n, k):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(n).astype(np.float32)
    assert list(oo.select_outliers(w, k)) == _brute_select(w, k)


def test_selection_ties_take_lower_indices():
    w = np.array([1.0, -3.0, 3.0, 0.0, 3.0, -3.0, 2.0, 0.0], dtype=np.float32)
    # four entries tie at |w| = 3: indices 1, 2, 4, 5
    assert list(oo.select_outliers(w, 2)) == [1, 2]
    assert list(oo.select_outliers(w, 5)) == [1, 2, 4, 5, 6]
    assert list(oo.select_outliers(w, 7)) == [0, 1, 2, 3, 4, 5, 6]  # the zeros tie too: lower index first
    assert list(oo.select_outliers(w, 7)) == _brute_select(w, 7)


def test_split_and_csr():
    rows, cols, k = 7, 96, 40
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float16)
    dense, idx, w32 = oo.split(w, "f16", rows, cols, k)
    assert np.array_equal(w32, w.astype(np.float32).reshape(-1))
    assert np.all(dense[idx] == 0) and np.array_equal(np.delete(dense, idx), np.delete(w32, idx))
    # every kept entry is at least as large as every dense entry
    assert np.abs(w32[idx]).min() >= np.abs(dense).max()
    row_ptr, col, val = oo.csr_of(idx, w32[idx], rows, cols)
    assert row_ptr[0] == 0 and row_ptr[-1] == k and np.all(np.diff(row_ptr) >= 0)
    for n in range(rows):
        seg = col[row_ptr[n]:row_ptr[n + 1]]
        assert np.all(np.diff(seg) > 0)
    S = oo.sparse_dense((row_ptr, col, val), rows, cols)
    assert np.array_equal(dense.astype(np.float64).reshape(rows, cols) + S, w.astype(np.float64))


def test_k_zero_is_the_plain_format():
    lin = workloads.tiny()
    q0, (rp, col, val) = oo.quantize_with_outliers(lin.W, "f32", 4, 256, 256, 0)
    q = oracle.quantize(lin.W.reshape(-1), "f32", 4)
    assert np.array_equal(q0.codes, q.codes) and np.array_equal(q0.absmax_q8, q.absmax_q8)
    assert np.array_equal(q0.absmax_c.view(np.uint32), q.absmax_c.view(np.uint32))
    assert rp[-1] == 0 and col.size == 0


def test_outliers_shrink_the_quantization_error():
    """The attention workload's planted x20 outliers: keeping them exact lowers both the largest
    and the typical dequantization error of the rest (they no longer stretch their blocks' scales)."""
    w = workloads.make_weight(2, 64, 1024, 0.02, "f16", outlier_frac=0.001)
    k = int(round(0.001 * w.size))
    plain = oracle.quantize(w.reshape(-1), "f16", 4)
    err_plain = np.abs(oracle.dequantize(plain.codes, plain.absmax_q8, plain.absmax_c, 4, w.size)
                       - w.astype(np.float32).reshape(-1))
    q, csr = oo.quantize_with_outliers(w, "f16", 4, 64, 1024, k)
    rec = oracle.dequantize(q.codes, q.absmax_q8, q.absmax_c, 4, w.size).astype(np.float64).reshape(64, 1024)
    rec = rec + oo.sparse_dense(csr, 64, 1024)
    err_split = np.abs(rec - w.astype(np.float64))
    assert err_split.max() < err_plain.max() and err_split.mean() < err_plain.mean()
    # at the outliers the residual restores w up to one float32 rounding of the residual
    idx = oo.select_outliers(w.astype(np.float32).reshape(-1), k)
    resid = np.abs(csr[2]).astype(np.float64)
    assert np.all(err_split.reshape(-1)[idx] <= resid * 2.0 ** -24)


def test_forward_merged_equals_unmerged():
    rows, cols, M, k = 6, 64, 3, 20
    rng = np.random.default_rng(5)
    w = rng.integers(-4, 5, size=(rows, cols)).astype(np.float32)
    x = rng.integers(-3, 4, size=(M, cols)).astype(np.float32)
    dense, idx, w32 = oo.split(w, "f32", rows, cols, k)
    csr = oo.csr_of(idx, w32[idx], rows, cols)
    y = oo.linear_outliers(x, "f32", dense.reshape(rows, cols), csr)
    assert np.array_equal(y, x.astype(np.float64) @ w.astype(np.float64).T)  # exact on small integers
    T = oo.linear_outliers_tolerance(x, "f32", dense.reshape(rows, cols), csr)
    assert np.all(np.abs(y) <= T)
