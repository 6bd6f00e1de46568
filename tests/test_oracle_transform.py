"""Pins for the oracle's orthogonal transform: sign pattern then normalised
Walsh-Hadamard (AXELRAM, arXiv 2604.02638, Abstract: orthogonal transform on
write, seeded sign pattern).  The dense matrix is checked against scipy's
Sylvester construction and the product against an independent butterfly
implementation written here."""

import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import axelram as A

DIMS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]


def butterfly_wht(x):
    """Unnormalised natural-order Walsh-Hadamard transform by butterflies."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


@pytest.mark.parametrize("d", DIMS)
def test_hadamard_is_sylvester(d):
    np.testing.assert_array_equal(A.sylvester_hadamard(d), hadamard(d))


def test_hadamard_small_cases():
    np.testing.assert_array_equal(A.sylvester_hadamard(2), [[1, 1], [1, -1]])
    h4 = A.sylvester_hadamard(4)
    h2 = A.sylvester_hadamard(2)
    np.testing.assert_array_equal(h4, np.block([[h2, h2], [h2, -h2]]))


@pytest.mark.parametrize("d", [2, 32, 128, 512])
def test_rotate_matches_butterflies(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((7, d))
    s = A.signs_from_bits(rng.integers(0, 2, d))
    np.testing.assert_allclose(A.rotate(x, s), butterfly_wht(s * x) / math.sqrt(d),
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("d", [2, 64, 128, 256, 512])
def test_orthogonality_and_inverse(d):
    rng = np.random.default_rng(3 + d)
    s = A.signs_from_bits(rng.integers(0, 2, d))
    h = A.sylvester_hadamard(d) / math.sqrt(d)
    eye = np.eye(d)
    # normalised WHT is symmetric and its own inverse; so is the sign flip
    np.testing.assert_allclose(h @ h, eye, atol=1e-14)
    np.testing.assert_allclose(np.diag(s) @ np.diag(s), eye, atol=0)
    t = A.rotate(eye, s)                      # row i = T e_i, so t.T is T
    tm = t.T
    np.testing.assert_allclose(tm.T @ tm, eye, atol=1e-13)
    # the composite T = H D / sqrt(d) is inverted by D H / sqrt(d)
    inv = np.diag(s) @ h
    np.testing.assert_allclose(inv @ tm, eye, atol=1e-13)
    x = rng.standard_normal((5, d))
    y = A.rotate(x, s)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                               rtol=1e-14)
    np.testing.assert_allclose((inv @ y.T).T, x, atol=1e-13)


def test_unit_vector_maps_to_flat_vector():
    d = 128
    rng = np.random.default_rng(5)
    s = A.signs_from_bits(rng.integers(0, 2, d))
    e0 = np.zeros(d)
    e0[0] = 1.0
    np.testing.assert_allclose(A.rotate(e0, s), s[0] * np.ones(d) / math.sqrt(d), atol=1e-15)


def test_transform_keys_normalises_and_keeps_norm():
    d = 128
    rng = np.random.default_rng(9)
    s = A.signs_from_bits(rng.integers(0, 2, d))
    k = rng.standard_normal((3, 4, d)) * 37.0
    k[1, 2] = 0.0                                         # zero key
    y, norms = A.transform_keys(k, s)
    np.testing.assert_allclose(norms, np.sqrt((k * k).sum(-1)), rtol=1e-15)
    unit = np.linalg.norm(y, axis=-1)
    assert unit[1, 2] == 0.0 and norms[1, 2] == 0.0
    mask = np.ones_like(unit, dtype=bool)
    mask[1, 2] = False
    np.testing.assert_allclose(unit[mask], 1.0, rtol=1e-14)
    np.testing.assert_allclose(y[0, 0], butterfly_wht(s * k[0, 0] / norms[0, 0]) / math.sqrt(d),
                               atol=1e-15)


def test_transformed_coordinates_have_variance_one_over_d():
    """For Gaussian keys the rotated unit vector is uniform on the sphere, so
    each coordinate has mean 0 and variance exactly 1/d, and is close to
    N(0, 1/d) for d = 128 (Kolmogorov-Smirnov at moderate sample size)."""
    from scipy import stats
    d = 128
    rng = np.random.default_rng(21)
    s = A.signs_from_bits(rng.integers(0, 2, d))
    k = rng.standard_normal((20000, d)) * np.exp(rng.standard_normal(d))  # outlier channels
    y, _ = A.transform_keys(k, s)
    np.testing.assert_allclose(np.mean(np.sum(y * y, axis=-1)), 1.0, rtol=1e-13)
    g = rng.standard_normal((20000, d))
    yg, _ = A.transform_keys(g, s)
    col = yg[:, 17] * math.sqrt(d)
    assert abs(col.mean()) < 5 / math.sqrt(len(col))
    assert abs(np.var(col) - 1.0) < 0.05
    assert stats.kstest(col, "norm").pvalue > 1e-3
