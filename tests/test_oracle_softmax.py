"""Pins of the oracle's softmax over score rows: it must equal scipy's
softmax and logsumexp on each row's tokens, sum to one, keep the ratio
p_t / p_t' = exp(scale (s_t - s_t')), ignore a constant added to a row, and
survive scores whose exponentials overflow float64."""

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import axelram as A


def _rows(seed, shape=(3, 4, 50), spread=5.0):
    return np.random.default_rng(seed).standard_normal(shape) * spread


@pytest.mark.parametrize("scale", [1.0, 1.0 / np.sqrt(128.0), 3.5])
def test_equals_scipy_on_each_prefix(scale):
    s = _rows(1)
    lens = np.array([50, 17, 1])
    p, lse = A.softmax_probs(s, lens, scale)
    for bi, n in enumerate(lens):
        ref = softmax(scale * s[bi, :, :n], axis=-1)
        np.testing.assert_allclose(p[bi, :, :n], ref, rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(lse[bi], logsumexp(scale * s[bi, :, :n], axis=-1), rtol=1e-14)
        assert np.all(np.isnan(p[bi, :, n:]))


def test_rows_sum_to_one_and_ratios():
    s = _rows(2)
    p, _ = A.softmax_probs(s, np.array([50, 50, 50]), 0.7)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=1e-14)
    r = p[..., 3] / p[..., 11]
    np.testing.assert_allclose(r, np.exp(0.7 * (s[..., 3] - s[..., 11])), rtol=1e-12)


def test_shift_invariance_and_single_token():
    s = _rows(3)
    lens = np.array([40, 1, 0])
    p1, l1 = A.softmax_probs(s, lens, 1.3)
    p2, l2 = A.softmax_probs(s + 17.0, lens, 1.3)
    np.testing.assert_allclose(p1[0, :, :40], p2[0, :, :40], rtol=1e-12)
    np.testing.assert_allclose(l2[0] - l1[0], 1.3 * 17.0, rtol=1e-12)
    assert np.all(p1[1, :, 0] == 1.0)
    np.testing.assert_allclose(l1[1], 1.3 * s[1, :, 0], rtol=1e-15)
    assert np.all(np.isinf(l1[2])) and np.all(l1[2] < 0) and np.all(np.isnan(p1[2]))


def test_large_scores_do_not_overflow():
    s = _rows(4, spread=1.0) + 2000.0                  # exp(2000) overflows float64
    p, lse = A.softmax_probs(s, np.array([50, 50, 50]), 1.0)
    assert np.all(np.isfinite(p)) and np.all(np.isfinite(lse))
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=1e-13)
