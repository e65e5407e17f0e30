"""Pins of the oracle's backward (gradients of the unmerged quantized-base + adapter layer).

The forward y = x W'^T + s (x A^T) B^T is linear in x, in A for fixed B and in B
for fixed A.  With small-integer inputs every float64 operation below is exact,
so for a unit perturbation e of one entry, <dy, y(. + e) - y(.)> computed with the
(separately pinned) forward oracle IS the gradient entry, with no rounding: that
brute force over every entry pins dx, dA and dB element by element.
"""
import numpy as np
import pytest

import oracle


def _ints(rng, shape, lo=-3, hi=4):
    return rng.integers(lo, hi, size=shape).astype(np.float32)


def _case(seed, M=2, N=3, K=5, r=2):
    rng = np.random.default_rng(seed)
    return (_ints(rng, (M, N)), _ints(rng, (M, K)), _ints(rng, (N, K)), _ints(rng, (r, K)),
            _ints(rng, (N, r)))


def _loss(dy, x, w, A, B, s):
    """<dy, y> in exact float64 arithmetic (integer inputs, power-of-two scale)."""
    y = oracle.linear(x, "f32", w, A, B, "f32", s)
    return float(np.sum(dy.astype(np.float64) * y))


@pytest.mark.parametrize("seed,s", [(0, 0.5), (1, 2.0), (2, -0.25)])
def test_every_entry_by_exact_differences(seed, s):
    dy, x, w, A, B = _case(seed)
    dx, dA, dB = oracle.linear_backward(dy, "f32", x, "f32", w, A, B, "f32", s)
    base = _loss(dy, x, w, A, B, s)
    for idx in np.ndindex(*x.shape):
        xp = x.copy()
        xp[idx] += 1
        assert _loss(dy, xp, w, A, B, s) - base == dx[idx]
    for idx in np.ndindex(*A.shape):
        Ap = A.copy()
        Ap[idx] += 1
        assert _loss(dy, x, w, Ap, B, s) - base == dA[idx]
    for idx in np.ndindex(*B.shape):
        Bp = B.copy()
        Bp[idx] += 1
        assert _loss(dy, x, w, A, Bp, s) - base == dB[idx]


def test_adjoint_identity_real_valued():
    """<dy, J v> = <grad, v> for a random direction v of each argument (float64 rounding only)."""
    rng = np.random.default_rng(7)
    M, N, K, r, s = 5, 9, 128, 3, 0.75
    dy = rng.standard_normal((M, N)).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = (rng.standard_normal((r, K)) / np.sqrt(K)).astype(np.float32)
    B = (rng.standard_normal((N, r)) * 0.01).astype(np.float32)
    dx, dA, dB = oracle.linear_backward(dy, "f32", x, "f32", w, A, B, "f32", s)
    g = dy.astype(np.float64)
    v = rng.standard_normal((M, K)).astype(np.float32)
    # y is linear in x with no offset: J_x v = y(v)
    lhs = np.sum(g * oracle.linear(v, "f32", w, A, B, "f32", s))
    assert np.isclose(lhs, np.sum(dx * v), rtol=1e-12, atol=0)
    # the adapter term is linear in A for fixed B, and in B for fixed A
    V = rng.standard_normal((r, K)).astype(np.float32)
    lhs = np.sum(g * (oracle.linear(x, "f32", w, V, B, "f32", s) - oracle.linear(x, "f32", w)))
    assert np.isclose(lhs, np.sum(dA * V), rtol=1e-10, atol=0)
    V = rng.standard_normal((N, r)).astype(np.float32)
    lhs = np.sum(g * (oracle.linear(x, "f32", w, A, V, "f32", s) - oracle.linear(x, "f32", w)))
    assert np.isclose(lhs, np.sum(dB * V), rtol=1e-10, atol=0)


def test_special_cases():
    dy, x, w, A, B = _case(3, M=3, N=4, K=6, r=2)
    base = dy.astype(np.float64) @ w.astype(np.float64)
    # no adapter: only the input gradient through the frozen base
    dx, dA, dB = oracle.linear_backward(dy, "f32", x, "f32", w)
    assert dA is None and dB is None and np.array_equal(dx, base)
    dx, dA, dB = oracle.linear_backward(dy, "f32", x, "f32", w, A[:0], B[:, :0], "f32", 1.0)
    assert dA is None and np.array_equal(dx, base)
    # scale 0: adapter gradients vanish
    dx, dA, dB = oracle.linear_backward(dy, "f32", x, "f32", w, A, B, "f32", 0.0)
    assert np.array_equal(dx, base) and not dA.any() and not dB.any()
    # B = 0 (the usual LoRA initialisation): dA = 0 and dx is the base term, but dB is not zero
    dx, dA, dB = oracle.linear_backward(dy, "f32", x, "f32", w, A, np.zeros_like(B), "f32", 2.0)
    assert np.array_equal(dx, base) and not dA.any()
    t = x.astype(np.float64) @ A.astype(np.float64).T
    assert dB.any() and np.array_equal(dB, 2.0 * (dy.astype(np.float64).T @ t))
    # M = 0: empty input gradient, zero adapter gradients
    dx, dA, dB = oracle.linear_backward(dy[:0], "f32", x[:0], "f32", w, A, B, "f32", 1.0)
    assert dx.shape == (0, 6) and not dA.any() and not dB.any()


def test_bf16_inputs_are_widened_exactly():
    rng = np.random.default_rng(4)
    dy, x, w, A, B = _case(4, M=2, N=3, K=8, r=2)
    # bf16 bit patterns of the same small integers (exact in bf16)
    to_bf16 = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ref = oracle.linear_backward(dy, "f32", x, "f32", w, A, B, "f32", 0.5)
    got = oracle.linear_backward(to_bf16(dy), "bf16", to_bf16(x), "bf16", w, to_bf16(A), to_bf16(B), "bf16", 0.5)
    for a, b in zip(ref, got):
        assert np.array_equal(a, b)
    del rng


def test_tolerance_sums_bound_and_are_tight_on_nonnegative_inputs():
    rng = np.random.default_rng(5)
    M, N, K, r, s = 4, 6, 64, 3, 1.25
    args = [rng.standard_normal(sh).astype(np.float32) for sh in ((M, N), (M, K), (N, K), (r, K), (N, r))]
    dy, x, w, A, B = args
    g = oracle.linear_backward(dy, "f32", x, "f32", w, A, B, "f32", -s)
    S = oracle.linear_backward_tolerance(dy, "f32", x, "f32", w, A, B, "f32", -s)
    for a, b in zip(g, S):
        assert np.all(np.abs(a) <= b * (1 + 1e-12))
    # all terms nonnegative: the magnitude sums are the gradients themselves
    pos = [np.abs(a) for a in args]
    g = oracle.linear_backward(pos[0], "f32", pos[1], "f32", pos[2], pos[3], pos[4], "f32", s)
    S = oracle.linear_backward_tolerance(pos[0], "f32", pos[1], "f32", pos[2], pos[3], pos[4], "f32", s)
    for a, b in zip(g, S):
        assert np.allclose(a, b, rtol=1e-13, atol=0)


def test_adapter_grads_alone_need_no_weight():
    """dA and dB do not involve W': the same values with any base weight, and from adapter_grads."""
    dy, x, w, A, B = _case(6, M=3, N=4, K=7, r=2)
    _, dA, dB = oracle.linear_backward(dy, "f32", x, "f32", w, A, B, "f32", 0.5)
    _, dA2, dB2 = oracle.linear_backward(dy, "f32", x, "f32", 3 * w + 1, A, B, "f32", 0.5)
    dA3, dB3 = oracle.adapter_grads(dy, "f32", x, "f32", A, B, "f32", 0.5)
    assert np.array_equal(dA, dA2) and np.array_equal(dB, dB2)
    assert np.array_equal(dA, dA3) and np.array_equal(dB, dB3)
    S = oracle.linear_backward_tolerance(dy, "f32", x, "f32", w, A, B, "f32", 0.5)
    S2 = oracle.adapter_grads_tolerance(dy, "f32", x, "f32", A, B, "f32", 0.5)
    assert np.array_equal(S[1], S2[0]) and np.array_equal(S[2], S2[1])


def test_column_restriction_of_the_input_gradient():
    """dx[:, ks] and dA[:, ks] only need the columns ks of W', A and x (what sampled checks use)."""
    rng = np.random.default_rng(8)
    M, N, K, r, s = 4, 6, 40, 3, 0.5
    dy, x, w, A, B = (rng.standard_normal(sh).astype(np.float32)
                      for sh in ((M, N), (M, K), (N, K), (r, K), (N, r)))
    full = oracle.linear_backward(dy, "f32", x, "f32", w, A, B, "f32", s)
    ks = [0, 7, 39]
    part = oracle.linear_backward(dy, "f32", x[:, ks], "f32", w[:, ks], A[:, ks], B, "f32", s)
    assert np.allclose(full[0][:, ks], part[0], rtol=1e-13, atol=0)
    assert np.allclose(full[1][:, ks], part[1], rtol=1e-13, atol=0)
