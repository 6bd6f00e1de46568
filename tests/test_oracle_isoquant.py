"""Pins of the oracle's block-rotation comparison transform ("IsoQuant:
Hardware-Aligned SO(4) Isoclinic Rotations for LLM KV Cache Compression",
Abstract: each 4-D block is a quaternion, T(v) = q_L v conj(q_R), one factor
for the Fast variant; 1,024 and 512 multiply-adds at d = 128).

* The Hamilton product satisfies i^2 = j^2 = k^2 = ijk = -1, ij = k = -ji and
  |ab| = |a||b|.
* Left and right multiplication by unit quaternions equal the 4x4 matrices
  written out by hand below; both are orthogonal with determinant +1, so T is
  in SO(4) on every block and preserves norms.
* The inverse is conj(q_L) w q_R.
* The write path is the plain definition and the multiply-add counts are the
  page's.
"""

import numpy as np
import pytest

from oracle import axelram as A
import workloads as W

ONE, I, J, K = np.eye(4)


def test_hamilton_units():
    m = A.quaternion_multiply
    for u in (I, J, K):
        np.testing.assert_array_equal(m(u, u), -ONE)
    np.testing.assert_array_equal(m(m(I, J), K), -ONE)
    np.testing.assert_array_equal(m(I, J), K)
    np.testing.assert_array_equal(m(J, I), -K)
    np.testing.assert_array_equal(m(J, K), I)
    np.testing.assert_array_equal(m(K, I), J)


def test_norm_is_multiplicative():
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal((2, 50, 4))
    np.testing.assert_allclose(np.linalg.norm(A.quaternion_multiply(a, b), axis=-1),
                               np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1), rtol=1e-13)


def _left_matrix(q):
    w, x, y, z = q
    return np.array([[w, -x, -y, -z], [x, w, -z, y], [y, z, w, -x], [z, -y, x, w]])


def _right_matrix(q):
    w, x, y, z = q
    return np.array([[w, -x, -y, -z], [x, w, z, -y], [y, -z, w, x], [z, y, -x, w]])


def test_products_equal_hand_written_matrices_in_so4():
    rng = np.random.default_rng(1)
    for _ in range(20):
        p, q, v = rng.standard_normal((3, 4))
        p /= np.linalg.norm(p)
        q /= np.linalg.norm(q)
        np.testing.assert_allclose(A.quaternion_multiply(p, v), _left_matrix(p) @ v, rtol=1e-13)
        np.testing.assert_allclose(A.quaternion_multiply(v, q), _right_matrix(q) @ v, rtol=1e-13)
        M = _left_matrix(p) @ _right_matrix(A.quaternion_conjugate(q))
        np.testing.assert_allclose(M @ M.T, np.eye(4), atol=1e-13)
        assert abs(np.linalg.det(M) - 1.0) < 1e-12


@pytest.mark.parametrize("full", [True, False])
def test_rotation_preserves_norms_and_inverts(full):
    d = 128
    rng = np.random.default_rng(2)
    qs = rng.standard_normal((d // 4, 2, 4))
    qs /= np.linalg.norm(qs, axis=-1, keepdims=True)
    ql, qr = qs[:, 0], (qs[:, 1] if full else None)
    x = rng.standard_normal((7, d))
    y = A.isoquant_rotate(x, ql, qr)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(A.isoquant_unrotate(y, ql, qr), x, atol=1e-13)
    # block m only mixes coordinates 4m .. 4m+3
    e = np.zeros(d)
    e[9] = 1.0
    assert np.count_nonzero(np.abs(A.isoquant_rotate(e, ql, qr)) > 1e-15) <= 4


def test_write_path_is_the_definition():
    d, b = 128, 3
    rng = np.random.default_rng(3)
    qs = W.isoquant_quaternions(d).astype(np.float64)
    keys = rng.standard_normal((5, d)) * 4.0
    keys[2] = 0.0
    w = A.isoquant_write_path(keys, qs[:, 0], qs[:, 1], b)
    c, t = A.lloyd_max_codebook(d, b)
    norms = np.linalg.norm(keys, axis=-1)
    for r in range(5):
        y = A.isoquant_rotate(keys[r] / norms[r], qs[:, 0], qs[:, 1]) if norms[r] else np.zeros(d)
        idx = np.array([np.sum(v > t) for v in y])
        np.testing.assert_array_equal(w["idx"][r], idx)
    assert np.all(w["idx"][2] == 3) and w["norms"][2] == 0.0


def test_fma_counts_match_the_page():
    assert A.rotation_fmas(128, "isoquant_full") == 1024
    assert A.rotation_fmas(128, "isoquant_fast") == 512
    assert A.rotation_fmas(128, "wht") == 0


def test_reconstruction_mse_of_gaussian_unit_vectors():
    # for i.i.d. Gaussian keys each rotated coordinate is close to N(0, 1/d),
    # so the per-vector error is close to d * D_b(1/d) = D_b(1) (Max's table)
    d, b = 128, 3
    rng = np.random.default_rng(4)
    keys = rng.standard_normal((4000, d))
    qs = W.isoquant_quaternions(d).astype(np.float64)
    c, _ = A.lloyd_max_codebook(d, b)
    for ql, qr in ((qs[:, 0], qs[:, 1]), (qs[:, 0], None)):
        w = A.isoquant_write_path(keys, ql, qr, b)
        mse = A.reconstruction_mse(keys, w["idx"], c, lambda y: A.isoquant_unrotate(y, ql, qr))
        assert abs(mse - 0.03455) < 0.003
