"""Pins of the oracle's quantile codebook (QLoRA page, NF4 codebook equation)."""
import math
import statistics

import numpy as np
import pytest

from oracle import normal_quantile, quantile_codebook

ALL_BITS = [1, 2, 3, 4, 5, 6, 7, 8]


def test_textbook_normal_quantiles(page_value):
    assert float(normal_quantile(0.75)) == pytest.approx(page_value("normal_quantile_0p75"), abs=1e-15)
    assert float(normal_quantile(0.975)) == pytest.approx(page_value("normal_quantile_0p975"), abs=1e-15)


def test_quantile_function_matches_stdlib():
    nd = statistics.NormalDist()
    for p in [1 / 1024, 0.01, 0.3, 0.5, 0.77, 0.999, 1023 / 1024]:
        assert abs(float(normal_quantile(p)) - nd.inv_cdf(p)) < 1e-14


def test_level_count_b4(page_value):
    assert quantile_codebook(4).size == int(page_value("codebook_levels_b4"))


@pytest.mark.parametrize("bits", ALL_BITS)
def test_invariants(bits):
    L = quantile_codebook(bits)
    n = 1 << bits
    assert L.dtype == np.float32 and L.size == n
    assert np.all(np.diff(L.astype(np.float64)) > 0)
    assert L[0] == -1.0 and L[-1] == 1.0
    assert np.array_equal(L.view(np.uint32), (-L[::-1]).view(np.uint32))  # mirror, bit-exact
    assert not np.any(L == 0.0)


def test_one_bit_is_sign():
    assert quantile_codebook(1).tolist() == [-1.0, 1.0]


@pytest.mark.parametrize("bits", ALL_BITS)
def test_levels_are_normalised_quantiles(bits):
    """Phi(L_i * z_max) == (i + 1/2) / 2^b, with Phi from erfc (independent of erfinv)."""
    L = quantile_codebook(bits)
    n = 1 << bits
    zmax = statistics.NormalDist().inv_cdf((n - 0.5) / n)
    for i, lv in enumerate(L):
        z = float(lv) * zmax
        phi = 0.5 * math.erfc(-z / math.sqrt(2.0))
        dens = math.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
        assert abs(phi - (i + 0.5) / n) <= dens * abs(z) * 2.0 ** -23 + 1e-15, (i, lv)


@pytest.mark.parametrize("bits", ALL_BITS)
def test_levels_rounded_to_nearest_f32(bits):
    """Each level is within half a float32 ulp of the real value z_i / z_max."""
    nd = statistics.NormalDist()
    L = quantile_codebook(bits)
    n = 1 << bits
    zmax = nd.inv_cdf((n - 0.5) / n)
    for i, lv in enumerate(L):
        exact = nd.inv_cdf((i + 0.5) / n) / zmax
        ulp = math.ulp(float(np.float32(abs(lv)))) * 2.0 ** 29  # float32 ulp via float64 ulp
        assert abs(float(lv) - exact) <= 0.5 * ulp * (1 + 1e-6) + 1e-15, (i, lv, exact)
