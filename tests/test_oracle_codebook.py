"""Pins for the oracle's Lloyd-Max codebook (design-time quantizer for
N(0, 1/d); AXELRAM, arXiv 2604.02638, Abstract).

The pins do not reuse the oracle's closed forms: conditional means and
distortions are recomputed by adaptive quadrature (scipy.integrate.quad) of
the Gaussian density, and the values are compared with Max's 1960 table."""

import math

import numpy as np
import pytest
from scipy import integrate

from oracle import axelram as A
from tests._golden import max1960_table

DIMS = [2, 8, 32, 128, 256, 512]
BITS = [1, 2, 3, 4]


def _pdf(sigma):
    return lambda x: math.exp(-0.5 * (x / sigma) ** 2) / (sigma * math.sqrt(2 * math.pi))


def _quad(f, lo, hi):
    val, _ = integrate.quad(f, lo, hi, epsabs=0.0, epsrel=1e-13, limit=200)
    return val


def quadrature_centroid_residual(d, c, t):
    """max_i |c_i - E[X | cell_i]| / sigma with the expectation by quadrature."""
    sigma = 1.0 / math.sqrt(d)
    p = _pdf(sigma)
    edges = [-math.inf] + list(t) + [math.inf]
    worst = 0.0
    for i, ci in enumerate(c):
        mass = _quad(p, edges[i], edges[i + 1])
        first = _quad(lambda x: x * p(x), edges[i], edges[i + 1])
        worst = max(worst, abs(ci - first / mass) / sigma)
    return worst


def quadrature_mse(d, c, t):
    sigma = 1.0 / math.sqrt(d)
    p = _pdf(sigma)
    edges = [-math.inf] + list(t) + [math.inf]
    return sum(_quad(lambda x, ci=ci: (x - ci) ** 2 * p(x), edges[i], edges[i + 1])
               for i, ci in enumerate(c))


def midpoint_residual(c, t):
    c, t = np.asarray(c), np.asarray(t)
    return float(np.max(np.abs(t - 0.5 * (c[:-1] + c[1:])))) if len(t) else 0.0


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("b", BITS)
def test_centroid_and_midpoint_conditions(d, b):
    c, t = A.lloyd_max_codebook(d, b)
    sigma = 1.0 / math.sqrt(d)
    assert len(c) == 2 ** b and len(t) == 2 ** b - 1
    assert quadrature_centroid_residual(d, c, t) <= 1e-11
    assert midpoint_residual(c, t) <= 1e-15 * sigma * 4
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    # symmetric density -> symmetric quantizer; 0 is a threshold
    np.testing.assert_allclose(c, -c[::-1], rtol=0, atol=1e-15 * sigma * 8)
    assert abs(t[len(t) // 2]) <= 1e-15 * sigma * 8


@pytest.mark.parametrize("d", DIMS)
def test_one_bit_closed_form(d):
    sigma = 1.0 / math.sqrt(d)
    c, t = A.lloyd_max_codebook(d, 1)
    expect = sigma * math.sqrt(2.0 / math.pi)
    np.testing.assert_allclose(c, [-expect, expect], rtol=1e-14, atol=0)
    assert abs(t[0]) < 1e-18
    assert abs(A.codebook_distortion(d, c, t) - sigma ** 2 * (1 - 2 / math.pi)) \
        <= 1e-14 * sigma ** 2


@pytest.mark.parametrize("b", BITS)
def test_matches_max_1960_table(b):
    table = max1960_table()[b]
    c, t = A.lloyd_max_codebook(1, b)          # d = 1: unit variance
    half = 2 ** (b - 1)
    np.testing.assert_allclose(c[half:], table["centroid"], rtol=6e-4, atol=6e-4)
    np.testing.assert_allclose(t[half - 1:], table["threshold"], rtol=6e-4, atol=6e-4)
    dist = A.codebook_distortion(1, c, t)
    assert abs(dist - table["distortion"][0]) <= 6e-4 * table["distortion"][0] + 1e-6


@pytest.mark.parametrize("d", [8, 128, 512])
@pytest.mark.parametrize("b", BITS)
def test_distortion_closed_form_matches_quadrature(d, b):
    c, t = A.lloyd_max_codebook(d, b)
    assert abs(A.codebook_distortion(d, c, t) - quadrature_mse(d, c, t)) \
        <= 1e-11 / d


@pytest.mark.parametrize("b", [2, 3, 4])
def test_codebook_is_a_local_minimum_of_mse(b):
    d = 128
    sigma = 1.0 / math.sqrt(d)
    c, t = A.lloyd_max_codebook(d, b)
    base = quadrature_mse(d, c, t)
    delta = 2e-3 * sigma
    for i in range(len(c)):
        for sgn in (-1.0, 1.0):
            cc = c.copy()
            cc[i] += sgn * delta
            assert quadrature_mse(d, cc, t) > base
    for i in range(len(t)):
        for sgn in (-1.0, 1.0):
            tt = t.copy()
            tt[i] += sgn * delta
            assert quadrature_mse(d, c, tt) > base


@pytest.mark.parametrize("b", [2, 3, 4])
def test_monte_carlo_distortion(b):
    d = 128
    rng = np.random.default_rng(11)
    x = rng.standard_normal(2_000_000) / math.sqrt(d)
    c, t = A.lloyd_max_codebook(d, b)
    err = (x - c[A.quantize(x, t)]) ** 2
    se = err.std() / math.sqrt(len(err))
    assert abs(err.mean() - A.codebook_distortion(d, c, t)) < 5 * se


def test_scale_equivariance():
    # the quantizer for N(0, 1/d) is the unit-variance one scaled by 1/sqrt(d)
    c1, t1 = A.lloyd_max_codebook(1, 3)
    c, t = A.lloyd_max_codebook(128, 3)
    np.testing.assert_allclose(c, c1 / math.sqrt(128), rtol=1e-13)
    np.testing.assert_allclose(t, t1 / math.sqrt(128), rtol=1e-13, atol=1e-17)
