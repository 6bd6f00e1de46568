"""Pins of the oracle's sign-pattern selection objective (AXELRAM, Abstract:
gradient-free selection over candidates and calibration samples; here with a
score-error stand-in for the perplexity objective).

* Negating the whole sign pattern mirrors every coordinate and the codebook is
  symmetric, so the objective of s and -s is the same.
* Scaling a calibration sample's keys by a positive constant (layer-wise norm
  heterogeneity) leaves the indices and the relative error unchanged.
* The exact scores equal einsum with query head h reading KV head h // G.
* The error equals the one from the independently pinned dequantize-then-dot
  path.
"""

import numpy as np
import pytest

from oracle import axelram as A
import workloads as W


def _data(seed=0, S=2, B=1, Hkv=2, Hq=4, T=48, d=32):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((S, B, Hkv, T, d)) * np.exp(rng.standard_normal(d)) + 0.7
    q = rng.standard_normal((S, B, Hq, d))
    return keys, q


def test_dense_scores_gqa_mapping():
    keys, q = _data()
    got = A.dense_scores(q[0], keys[0])
    G = q.shape[2] // keys.shape[2]
    kk = np.repeat(keys[0], G, axis=1)                  # head h -> KV head h // G
    np.testing.assert_allclose(got, np.einsum("bhd,bhtd->bht", q[0], kk), rtol=1e-13)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_negated_pattern_has_the_same_objective(b):
    keys, q = _data(1)
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2, size=(2, 32)).astype(np.uint8)
    cands = np.concatenate([bits, 1 - bits])
    e = A.sign_selection_errors(keys, q, cands, b)
    np.testing.assert_allclose(e[:2], e[2:], rtol=1e-9)


def test_sample_scale_does_not_change_relative_error():
    keys, q = _data(2)
    cands = np.random.default_rng(6).integers(0, 2, size=(3, 32)).astype(np.uint8)
    e1 = A.sign_selection_errors(keys, q, cands, 3)
    keys2 = keys.copy()
    keys2[1] *= 37.5
    e2 = A.sign_selection_errors(keys2, q, cands, 3)
    r1 = e1[..., 0] / e1[..., 1]
    r2 = e2[..., 0] / e2[..., 1]
    np.testing.assert_allclose(r1, r2, rtol=1e-10)
    assert A.select_sign_pattern(e1)[0] == A.select_sign_pattern(e2)[0]


def test_error_matches_dequantize_then_dot():
    keys, q = _data(3, S=1)
    bits = np.random.default_rng(7).integers(0, 2, size=(1, 32)).astype(np.uint8)
    b = 3
    e = A.sign_selection_errors(keys, q, bits, b)
    s = A.signs_from_bits(bits[0])
    c, t = A.lloyd_max_codebook(32, b)
    y, norms = A.transform_keys(keys[0], s)
    idx = A.quantize(y, t)
    deq = A.dequantize_then_dot(q[0], idx, norms, s, c)
    exact = np.einsum("bhd,bhtd->bht", q[0], np.repeat(keys[0], 2, axis=1))
    np.testing.assert_allclose(e[0, 0, 0], np.sum((deq - exact) ** 2), rtol=1e-10)
    np.testing.assert_allclose(e[0, 0, 1], np.sum(exact ** 2), rtol=1e-12)


def test_selection_takes_the_best_worst_case():
    err = np.array([[[4.0, 1.0], [1.0, 1.0]],       # worst sample sqrt(4) = 2
                    [[1.0, 1.0], [2.25, 1.0]],      # worst 1.5
                    [[0.01, 1.0], [9.0, 1.0]]])     # worst 3
    idx, obj = A.select_sign_pattern(err)
    assert idx == 1
    np.testing.assert_allclose(obj, [2.0, 1.5, 3.0])


def test_selection_zero_reference_and_ties():
    """A sample with no exact score mass counts 0 if its table scores are zero
    too and +inf otherwise; equal objectives go to the first candidate."""
    err = np.array([[[0.0, 0.0], [1.0, 4.0]],       # worst max(0, 0.5) = 0.5
                    [[1e-30, 0.0], [0.0, 1.0]],     # inf
                    [[0.25, 1.0], [0.0, 9.0]]])     # worst 0.5: ties with 0
    idx, obj = A.select_sign_pattern(err)
    assert idx == 0
    assert obj[0] == 0.5 and obj[1] == np.inf and obj[2] == 0.5


@pytest.mark.parametrize("bad", [np.nan, -1.0])
def test_selection_rejects_bad_sums(bad):
    err = np.ones((2, 2, 2))
    err[1, 0, 1] = bad
    with pytest.raises(ValueError):
        A.select_sign_pattern(err)


def test_calibration_generator_shapes_and_candidates():
    cal = W.calibration_samples(count=3, T=16)
    assert tuple(cal["keys"].shape) == (3, 1, 2, 16, 128)
    assert tuple(cal["q"].shape) == (3, 1, 16, 128)
    cands = W.sign_candidates(128, count=5)
    assert np.array_equal(cands[0], W.sign_bits(128))
    assert len({c.tobytes() for c in cands}) == 5
