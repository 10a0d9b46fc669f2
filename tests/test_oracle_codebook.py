"""Pins for the Lloyd-Max codebook solver."""
import math

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import codebook
from tests.conftest import load_golden


def beta_density(t, d):
    """Coordinate law from scipy's Beta distribution: (t+1)/2 ~ Beta(a, a)."""
    a = (d - 1) / 2
    return stats.beta(a, a).pdf((np.asarray(t) + 1) / 2) / 2


@pytest.mark.parametrize("d", [8, 64, 128])
def test_density_matches_beta_law_and_normalises(d):
    ts = np.linspace(-0.95, 0.95, 41)
    assert np.allclose(codebook.density(ts, d), beta_density(ts, d), rtol=1e-10, atol=1e-300)
    total, _ = integrate.quad(lambda t: codebook.density(t, d), -1, 1, epsabs=1e-14)
    assert abs(total - 1) < 1e-10


@pytest.mark.parametrize("d,bits", [(128, 1), (128, 2), (128, 3), (128, 4), (128, 7), (64, 3), (32, 2)])
def test_lloyd_max_conditions_by_independent_quadrature(d, bits):
    c, t = codebook.codebook(d, bits)
    n = 1 << bits
    assert len(c) == n and len(t) == n - 1
    assert np.all(np.diff(c) > 0)
    # boundaries are midpoints, codebook odd-symmetric, middle boundary 0
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-16)
    assert np.array_equal(c, -c[::-1])
    assert t[n // 2 - 1] == 0.0
    # centroid = conditional mean of its cell, by adaptive quadrature of scipy's
    # Beta density (not the solver's closed forms)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(n):
        lo, hi = edges[k], edges[k + 1]
        pts = [x for x in (-0.5, 0.0, 0.5) if lo < x < hi]
        m0, _ = integrate.quad(lambda x: beta_density(x, d), lo, hi, epsabs=1e-15, epsrel=1e-13,
                               points=pts or None, limit=200)
        m1, _ = integrate.quad(lambda x: x * beta_density(x, d), lo, hi, epsabs=1e-15, epsrel=1e-13,
                               points=pts or None, limit=200)
        assert abs(m1 / m0 - c[k]) < 1e-12, (k, m1 / m0, c[k])


def test_one_bit_closed_form():
    # 1 bit: c = +-E|t| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    for d in (16, 128, 256):
        c, t = codebook.codebook(d, 1)
        e_abs = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
        assert abs(c[1] - e_abs) < 1e-14 and c[0] == -c[1] and t[0] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_high_dimension_limit_is_max_gaussian_quantizer(bits):
    g = load_golden("max1960_gaussian_quantizer.json")["quantizers"][str(bits)]
    d = 40000
    c, t = codebook.lloyd_max(d, bits)[:2]
    n = 1 << bits
    pos_c = np.sqrt(d) * c[n // 2:]
    pos_t = np.sqrt(d) * t[n // 2 - 1:]
    assert np.allclose(pos_c, g["outputs"], rtol=2e-3, atol=2e-3)
    assert np.allclose(pos_t, g["boundaries"], rtol=2e-3, atol=2e-3)
    mse = d * codebook.coordinate_mse(c, t, d)
    assert abs(mse - g["mse"]) < 3e-3 * g["mse"] + 1e-4


def test_codebook_is_a_local_minimum_of_distortion():
    d, bits = 128, 3
    c, t = codebook.codebook(d, bits)

    def distortion(cc, tt):
        edges = np.concatenate(([-1.0], tt, [1.0]))
        tot = 0.0
        for k in range(len(cc)):
            v, _ = integrate.quad(lambda x: (x - cc[k]) ** 2 * beta_density(x, d), edges[k], edges[k + 1],
                                  epsabs=1e-16, epsrel=1e-12, limit=200)
            tot += v
        return tot

    base = distortion(c, t)
    assert abs(base - codebook.coordinate_mse(c, t, d)) < 1e-12
    for k, eps in ((0, 1e-3), (3, -1e-3), (5, 2e-3)):
        cc = c.copy()
        cc[k] += eps
        assert distortion(cc, t) > base
    tt = t.copy()
    tt[2] += 1e-3
    assert distortion(c, tt) > base


def test_distortion_falls_with_bits():
    d = 128
    mses = [d * codebook.coordinate_mse(*codebook.codebook(d, b), d) for b in (1, 2, 3, 4)]
    assert all(a > b for a, b in zip(mses, mses[1:]))
    # Each extra bit buys close to the high-resolution 6 dB (x4) at 3-4 bits.
    assert 3.0 < mses[2] / mses[3] < 4.2


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_table_centroids_are_fp32_and_cost_nothing(bits):
    """The table reconstruction values are the fp32 roundings of the exact
    centroids: representable in fp32, still antisymmetric, within half an fp32
    ulp of the exact values, and their distortion (independent quadrature,
    exact boundaries) equals the optimum to 1e-12 of it."""
    d = 128
    c, t = codebook.codebook(d, bits)
    cs, ts = codebook.table_codebook(d, bits)
    assert np.array_equal(ts, t)
    assert np.array_equal(cs.astype(np.float32).astype(np.float64), cs)
    assert np.array_equal(cs, -cs[::-1])
    ulp = np.spacing(np.abs(c).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(cs - c) <= 0.5 * ulp)

    def distortion(cc):
        edges = np.concatenate(([-1.0], t, [1.0]))
        tot = 0.0
        for k in range(len(cc)):
            v, _ = integrate.quad(lambda x: (x - cc[k]) ** 2 * beta_density(x, d), edges[k], edges[k + 1],
                                  epsabs=1e-16, epsrel=1e-12, limit=200)
            tot += v
        return tot

    base, table = distortion(c), distortion(cs)
    assert base <= table * (1 + 1e-12) and table < base * (1 + 1e-10)
