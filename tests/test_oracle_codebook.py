"""Pins of the oracle's Lloyd-Max codebook (CPU only)."""
import math

import numpy as np
import pytest
from scipy import integrate, special

from conftest import read_golden
from oracle import codebook as cbm


@pytest.mark.parametrize("d", [16, 128, 1024])
def test_one_bit_closed_form(d):
    # One bit: the centroids are +-E|X| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).
    cb = cbm.lloyd_max(d, 1)
    e_abs = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert cb.centroids[1] == pytest.approx(e_abs, rel=1e-13)
    assert cb.centroids[0] == -cb.centroids[1]
    assert cb.boundaries[0] == 0.0
    if d == 128:
        assert cb.centroids[1] == pytest.approx(0.0706616, abs=5e-8)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_d3_is_uniform_quantizer(bits):
    # For d = 3 the coordinate is uniform on [-1, 1] (Archimedes), whose
    # Lloyd-Max quantizer is the uniform one with MSE (2/L)^2 / 12.
    L = 1 << bits
    cb = cbm.lloyd_max(3, bits)
    j = np.arange(L)
    assert np.allclose(cb.centroids, -1 + (2 * j + 1) / L, atol=1e-13)
    assert np.allclose(cb.boundaries, -1 + 2 * j[1:] / L, atol=1e-13)
    assert cbm.mse(cb) == pytest.approx((2.0 / L) ** 2 / 12.0, rel=1e-10)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_fixed_point_conditions_by_quadrature(bits):
    # Centroid condition checked with adaptive quadrature, independent of the
    # closed-form mass / first moment used by the iteration.
    d = 128
    cb = cbm.lloyd_max(d, bits)
    edges = np.concatenate(([-1.0], cb.boundaries, [1.0]))
    f = lambda x: cbm.density(x, d)
    for jj in range(cb.levels):
        a, b = edges[jj], edges[jj + 1]
        mass = integrate.quad(f, a, b, epsabs=0, epsrel=1e-13, limit=200)[0]
        mom = integrate.quad(lambda x: x * f(x), a, b, epsabs=0, epsrel=1e-13, limit=200)[0]
        assert cb.centroids[jj] == pytest.approx(mom / mass, rel=1e-9, abs=1e-12)
    assert np.allclose(cb.boundaries, 0.5 * (cb.centroids[:-1] + cb.centroids[1:]), atol=1e-15)
    assert np.all(np.diff(cb.centroids) > 0)
    assert np.array_equal(cb.centroids, -cb.centroids[::-1])


def test_density_normalised():
    for d in (3, 16, 128):
        assert integrate.quad(lambda x: cbm.density(x, d), -1, 1, epsrel=1e-13)[0] == pytest.approx(1.0, rel=1e-12)
        # second moment of a coordinate of a unit vector is 1/d
        m2 = integrate.quad(lambda x: x * x * cbm.density(x, d), -1, 1, epsrel=1e-13)[0]
        assert m2 == pytest.approx(1.0 / d, rel=1e-12)


def test_large_d_tends_to_max_gaussian_levels():
    d = 20000
    for row in read_golden("max1960_gaussian_levels.txt"):
        bits, mse_max = int(row[0]), float(row[1])
        levels = np.array([float(v) for v in row[2:]])
        cb = cbm.lloyd_max(d, bits)
        scaled = math.sqrt(d) * cb.centroids[cb.levels // 2:]
        assert np.allclose(scaled, levels, atol=1.5e-3), (bits, scaled, levels)
        assert cbm.distortion(cb) == pytest.approx(mse_max, rel=3e-3)


def test_distortion_within_pages_factor_and_above_minimum():
    factor = float([r for r in read_golden("pages_figures.txt") if r[0] == "distortion_factor"][0][1])
    for bits in (1, 2, 3, 4):
        D = cbm.distortion(cbm.lloyd_max(128, bits))
        assert 4.0 ** -bits <= D <= math.sqrt(3) * math.pi / 2 * 4.0 ** -bits
        # the page's rounded factor: within about 2.7x of the minimum
        assert D / 4.0 ** -bits < factor + 0.05


def test_cosine_matches_pages():
    for row in read_golden("pages_figures.txt"):
        if row[0] != "cosine":
            continue
        bits, cos = int(row[1]), float(row[2])
        D = cbm.distortion(cbm.lloyd_max(128, bits))
        assert round(math.sqrt(1 - D), 3) == cos


def test_distortion_ratio_per_bit():
    D = [cbm.distortion(cbm.lloyd_max(128, b)) for b in (1, 2, 3, 4)]
    for a, b in zip(D, D[1:]):
        assert 3.0 < a / b < 4.2


def test_mse_identity_with_centroid_energy():
    # At the fixed point, d*MSE = 1 - d * sum_j P_j c_j^2.
    for bits in (2, 4):
        cb = cbm.lloyd_max(128, bits)
        edges = np.concatenate(([-1.0], cb.boundaries, [1.0]))
        P = cbm.cell_mass(edges[:-1], edges[1:], 128)
        assert cbm.distortion(cb) == pytest.approx(1 - 128 * np.sum(P * cb.centroids ** 2), rel=1e-9)


def test_eight_bit_distortion_matches_high_resolution_formula():
    """At 256 levels the optimum approaches the Panter-Dite high-resolution
    distortion (1 / (12 L^2)) (integral of f^(1/3))^3 per coordinate (Panter
    and Dite 1951; Gersho and Gray, "Vector Quantization and Signal
    Compression", section 6.3), evaluated here by quadrature of the
    coordinate density; the iteration never sees this formula."""
    d, L = 128, 256
    g = integrate.quad(lambda x: cbm.density(x, d) ** (1.0 / 3.0), -1, 1, epsabs=0, epsrel=1e-12, limit=400)[0]
    pd = g ** 3 / (12 * L * L)
    cb = cbm.lloyd_max(d, 8)
    assert cbm.distortion(cb) == pytest.approx(d * pd, rel=0.01)
    # and a quarter of the 7-bit distortion, as the formula's 4^-b scaling says
    ratio = cbm.distortion(cbm.lloyd_max(d, 7)) / cbm.distortion(cb)
    assert 3.9 < ratio < 4.1
