"""Pins of the oracle's double-binary adapter branch (LoRDBA page, section 2)."""
import math

import numpy as np
import pytest

import oracle
from oracle import dba


def _signs(rng, shape):
    return np.where(rng.integers(0, 2, size=shape) == 1, 1.0, -1.0)


def _case(seed, M=3, N=5, K=7, R=4, l=1, ints=True):
    rng = np.random.default_rng(seed)
    if ints:
        draw = lambda sh: rng.integers(-3, 4, size=sh).astype(np.float64)
    else:
        draw = lambda sh: rng.standard_normal(sh).astype(np.float16).astype(np.float64)
    x = draw((M, K)).astype(np.float32)
    w = draw((N, K)).astype(np.float32)
    al, be, ga = draw((l, N)), draw((l, R)), draw((l, K))
    S1, S2 = _signs(rng, (N, R)), _signs(rng, (R, K))
    return x, w, al, be, ga, S1, S2


@pytest.mark.parametrize("shape", [(5, 4), (3, 32), (2, 33), (4, 70)])
def test_pack_round_trip_and_bit_order(shape):
    rng = np.random.default_rng(sum(shape))
    S = _signs(rng, shape)
    P = dba.pack_signs(S)
    assert P.dtype == np.uint32 and P.shape == (shape[0], (shape[1] + 31) // 32)
    assert np.array_equal(dba.unpack_signs(P, shape[1]), S)
    # bit c of the row's little-endian bit string is entry c (via Python integers)
    for r in range(shape[0]):
        big = sum(int(P[r, i]) << (32 * i) for i in range(P.shape[1]))
        for c in range(shape[1]):
            assert ((big >> c) & 1) == (1 if S[r, c] > 0 else 0)
        assert big >> shape[1] == 0  # padding bits are zero


@pytest.mark.parametrize("seed,l", [(0, 1), (1, 1), (2, 2), (3, 3)])
def test_equals_the_lora_form_exactly(seed, l):
    """With A = [B2 diag(gamma_i)]_i stacked and B = [diag(alpha_i) B1 diag(beta_i)]_i, the branch
    is a rank-lR LoRA branch with scale 1: the (separately pinned) forward oracle gives the same
    values, exactly on small-integer inputs."""
    x, w, al, be, ga, S1, S2 = _case(seed, l=l)
    y = dba.linear_dba(x, "f32", w, al, be, ga, dba.pack_signs(S1), dba.pack_signs(S2))
    A = np.concatenate([S2 * ga[i][None, :] for i in range(l)], axis=0)
    B = np.concatenate([al[i][:, None] * S1 * be[i][None, :] for i in range(l)], axis=1)
    ref = oracle.linear(x, "f32", w, A.astype(np.float32), B.astype(np.float32), "f32", 1.0)
    assert np.array_equal(y, ref)


def test_add_subtract_form_brute_force():
    """The page's multiplication-free form: each stage-1 entry is the sum over k with sign +1
    minus the sum over k with sign -1 (exact sums with math.fsum)."""
    x, w, al, be, ga, S1, S2 = _case(4, M=2, N=3, K=9, R=5, l=2, ints=False)
    y = dba.linear_dba(x, "f32", w, al, be, ga, dba.pack_signs(S1), dba.pack_signs(S2))
    base = x.astype(np.float64) @ w.astype(np.float64).T
    for m in range(2):
        for n in range(3):
            terms = []
            for i in range(2):
                for j in range(5):
                    xg = [float(x[m, k]) * ga[i, k] for k in range(9)]
                    z = math.fsum(v for v, s in zip(xg, S2[j]) if s > 0) - math.fsum(v for v, s in zip(xg, S2[j]) if s < 0)
                    terms.append(al[i, n] * (z * be[i, j] if S1[n, j] > 0 else -z * be[i, j]))
            ref = math.fsum(terms)
            assert abs((y[m, n] - base[m, n]) - ref) <= 1e-12 * (abs(ref) + 1e-6)


def test_delta_w_merged_equals_unmerged():
    x, w, al, be, ga, S1, S2 = _case(5, M=4, N=6, K=10, R=3, l=2)
    P1, P2 = dba.pack_signs(S1), dba.pack_signs(S2)
    dW = dba.delta_w(al, be, ga, P1, P2)
    y = dba.linear_dba(x, "f32", w, al, be, ga, P1, P2)
    merged = x.astype(np.float64) @ (w.astype(np.float64) + dW).T
    assert np.array_equal(y, merged)
    # all-ones scales and l = 1: dW is the integer product of the sign factors
    one = lambda n: np.ones((1, n))
    assert np.array_equal(dba.delta_w(one(6), one(3), one(10), P1, P2), S1 @ S2)


def test_zero_scale_gives_the_base():
    x, w, al, be, ga, S1, S2 = _case(6)
    base = oracle.linear(x, "f32", w)
    for z in ("alpha", "beta", "gamma"):
        args = {"alpha": al, "beta": be, "gamma": ga}
        args[z] = np.zeros_like(args[z])
        y = dba.linear_dba(x, "f32", w, args["alpha"], args["beta"], args["gamma"],
                           dba.pack_signs(S1), dba.pack_signs(S2))
        assert np.array_equal(y, base)


def test_tolerance_sums():
    x, w, al, be, ga, S1, S2 = _case(7, ints=False, l=2)
    P1, P2 = dba.pack_signs(S1), dba.pack_signs(S2)
    y = dba.linear_dba(x, "f32", w, al, be, ga, P1, P2)
    S = dba.linear_dba_tolerance(x, "f32", w, al, be, ga, P1, P2)
    assert np.all(np.abs(y) <= S * (1 + 1e-12))
    # nonnegative values and all-plus signs: the sums are the result itself
    pos = lambda a: np.abs(a)
    ones1, ones2 = np.ones_like(S1), np.ones_like(S2)
    y = dba.linear_dba(pos(x), "f32", pos(w), pos(al), pos(be), pos(ga), dba.pack_signs(ones1), dba.pack_signs(ones2))
    S = dba.linear_dba_tolerance(pos(x), "f32", pos(w), pos(al), pos(be), pos(ga), dba.pack_signs(ones1),
                                 dba.pack_signs(ones2))
    assert np.allclose(y, S, rtol=1e-13, atol=0)


def test_page_storage_arithmetic():
    """LoRDBA page: one bit per sign-factor entry plus fp16 scales; at most 4 bits per adapter
    parameter (section 5), and about 10.6x smaller than the fp16 LoRA factors of the same shape
    (section 4, RQ2) -- here at N = K = 4096 with l = 1 that ratio is reached at R = 32."""
    N = K = 4096
    for R in (8, 16, 32, 64):
        bits = dba.adapter_bits(N, K, R, 1)
        assert bits / (R * (N + K)) <= 4.0
    ratio = lambda R: 16 * R * (N + K) / dba.adapter_bits(N, K, R, 1)
    assert abs(ratio(32) - 10.6) < 0.1
    assert ratio(64) > ratio(32) > ratio(16) > 1
