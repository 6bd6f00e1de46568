"""Pins for the oracle's small helpers that the rest builds on.

The normal cell mass feeds the Lloyd-Max centroid condition ("AXELRAM:
Quantize Once, Never Dequantize", Abstract: the codebook is Lloyd-Max for
N(0, 1/d)); the key norm is the stored per-key scale the same abstract names.
"""

import math

import numpy as np
import pytest
from scipy import special, stats

from oracle import axelram as A


def test_cell_mass_closed_forms():
    inf = math.inf
    assert A.gaussian_cell_mass(-inf, inf) == pytest.approx(1.0, abs=1e-15)
    assert A.gaussian_cell_mass(0.0, inf) == pytest.approx(0.5, abs=1e-16)
    assert A.gaussian_cell_mass(-inf, 0.0) == pytest.approx(0.5, abs=1e-16)
    # P(|Z| <= 1) = erf(1 / sqrt 2)
    assert A.gaussian_cell_mass(-1.0, 1.0) == pytest.approx(0.6826894921370859, rel=1e-14)
    # far tail Q(8), where 1 - Phi(8) would cancel to nothing
    assert A.gaussian_cell_mass(8.0, inf) == pytest.approx(6.220960574271785e-16, rel=1e-12)
    assert A.gaussian_cell_mass(-inf, -8.0) == pytest.approx(6.220960574271785e-16, rel=1e-12)


def test_cell_mass_symmetry_additivity_and_library():
    rng = np.random.default_rng(11)
    for _ in range(200):
        a, b, c = np.sort(rng.uniform(-6.0, 6.0, 3))
        m_ab, m_bc = A.gaussian_cell_mass(a, b), A.gaussian_cell_mass(b, c)
        assert A.gaussian_cell_mass(-b, -a) == pytest.approx(m_ab, rel=1e-12, abs=1e-300)
        assert m_ab + m_bc == pytest.approx(A.gaussian_cell_mass(a, c), rel=1e-12)
        # the survival function keeps relative accuracy in either tail
        ref = (stats.norm.sf(a) - stats.norm.sf(b)) if a >= 0 else (
            (stats.norm.cdf(b) - stats.norm.cdf(a)) if b <= 0 else
            0.5 * (special.erf(b / math.sqrt(2)) - special.erf(a / math.sqrt(2))))
        assert m_ab == pytest.approx(ref, rel=1e-10, abs=1e-300)


def test_cell_mean_is_the_truncated_normal_mean():
    for lo, hi in ((-1.0, 0.5), (0.3, 2.0), (-math.inf, -1.2), (1.5, math.inf)):
        ref = stats.truncnorm.mean(lo, hi)
        assert A.gaussian_cell_mean(lo, hi) == pytest.approx(ref, rel=1e-10)


def test_key_norms():
    assert A.key_norms(np.array([3.0, 4.0])) == pytest.approx(5.0, abs=0.0)
    eye = np.eye(128)
    assert np.array_equal(A.key_norms(eye), np.ones(128))
    assert A.key_norms(np.ones(512)) == pytest.approx(math.sqrt(512), rel=1e-15)
    rng = np.random.default_rng(12)
    k = rng.standard_normal((3, 5, 256))
    n = A.key_norms(k)
    assert n.shape == (3, 5)
    assert np.allclose(A.key_norms(-2.5 * k), 2.5 * n, rtol=1e-14)
    assert np.allclose(n, np.linalg.norm(k, axis=-1), rtol=1e-14)
    # fp16 input is upcast before squaring (fp16 squares would overflow here)
    big = np.full(128, 1000.0, dtype=np.float16)
    assert A.key_norms(big) == pytest.approx(1000.0 * math.sqrt(128), rel=1e-12)
