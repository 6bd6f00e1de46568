"""Pins for the oracle's read path: table lookup with no inverse transform
(AXELRAM, arXiv 2604.02638, Abstract) against dequantize-then-dot computed
independently here, and the page's 102.4x multiplication figure."""

import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import axelram as A
from tests._golden import abstract_figures


def _case(seed, B=2, Hkv=2, G=3, T=9, d=32, b=3):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2, d)
    keys = rng.standard_normal((B, Hkv, T, d)) * np.exp(rng.standard_normal(d))
    q = rng.standard_normal((B, Hkv * G, d))
    return keys, q, bits, b


def independent_dequantize_dot(q, idx, norms, bits, centroids):
    """k~ = ||k|| * D H c[idx] / sqrt(d) in key space, score = q . k~."""
    d = q.shape[-1]
    s = np.where(np.asarray(bits) != 0, -1.0, 1.0)
    h = hadamard(d).astype(np.float64)
    k_rec = np.einsum("ij,...j->...i", h, centroids[idx]) / math.sqrt(d)
    k_rec = k_rec * s * norms[..., None]
    G = q.shape[1] // idx.shape[1]
    out = np.zeros((q.shape[0], q.shape[1], idx.shape[2]))
    for bi in range(q.shape[0]):
        for h_ in range(q.shape[1]):
            for t in range(idx.shape[2]):
                out[bi, h_, t] = sum(q[bi, h_, j] * k_rec[bi, h_ // G, t, j] for j in range(d))
    return out


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [32, 64])
def test_lut_score_equals_dequantize_then_dot(b, d):
    keys, q, bits, _ = _case(b * 10 + d, d=d, b=b)
    s = A.signs_from_bits(bits)
    w = A.write_path(keys, s, b)
    c, _ = A.lloyd_max_codebook(d, b)
    got = A.read_path(q, w["packed"], w["norms"], s, b)
    ref = independent_dequantize_dot(q, w["idx"], w["norms"], bits, c)
    cond = A.score_condition(A.transform_queries(q, s), w["idx"], w["norms"], c)
    assert np.all(np.abs(got - ref) <= 1e-12 * cond + 1e-300)
    # and the oracle's own long-way routine agrees too
    np.testing.assert_allclose(A.dequantize_then_dot(q, w["idx"], w["norms"], s, c), ref,
                               rtol=0, atol=1e-12 * cond.max())


def test_rotated_domain_dot():
    keys, q, bits, b = _case(5)
    s = A.signs_from_bits(bits)
    w = A.write_path(keys, s, b)
    c, _ = A.lloyd_max_codebook(keys.shape[-1], b)
    qp = A.transform_queries(q, s)
    got = A.lut_scores(qp, w["idx"], w["norms"], c)
    G = q.shape[1] // keys.shape[1]
    for bi in range(q.shape[0]):
        for h in range(q.shape[1]):
            ref = w["norms"][bi, h // G] * (c[w["idx"][bi, h // G]] @ qp[bi, h])
            np.testing.assert_allclose(got[bi, h], ref, rtol=1e-13, atol=1e-13)


def test_gqa_head_mapping():
    keys, q, bits, b = _case(6, Hkv=2, G=2)
    keys[:, 1] = 0.0                                  # KV head 1 is empty
    s = A.signs_from_bits(bits)
    w = A.write_path(keys, s, b)
    sc = A.read_path(q, w["packed"], w["norms"], s, b)
    assert np.all(sc[:, 2:] == 0.0)                   # heads 2, 3 read KV head 1
    assert np.all(np.abs(sc[:, :2]) > 0.0)


def test_quantized_score_approximates_exact_dot():
    """With many keys the quantization error of the score has variance close
    to ||k||^2 * sum_j q'_j^2 * E[(y_j - c(y_j))^2], i.e. ||k||^2 ||q||^2 D_b."""
    d, b = 128, 3
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 2, d)
    s = A.signs_from_bits(bits)
    keys = rng.standard_normal((1, 1, 20000, d))
    q = rng.standard_normal((1, 1, d))
    w = A.write_path(keys, s, b)
    sc = A.read_path(q, w["packed"], w["norms"], s, b)[0, 0]
    exact = keys[0, 0] @ q[0, 0]
    c, t = A.lloyd_max_codebook(d, b)
    per_coord = A.codebook_distortion(d, c, t)
    expect = np.mean(w["norms"][0, 0] ** 2) * (q[0, 0] @ q[0, 0]) * per_coord
    rel = np.var(sc - exact) / expect
    assert 0.85 < rel < 1.15


def test_multiplication_reduction_figure():
    fig = abstract_figures()["multiplication_reduction"]
    dense, table, ratio = A.multiplications_per_query(4096, 128, 3)
    assert dense == 524288 and table == 5120
    assert ratio == fig


def test_empty_inputs():
    d, b = 32, 2
    s = np.ones(d)
    w = A.write_path(np.zeros((1, 1, 0, d)), s, b)
    assert w["packed"].shape == (1, 1, 0, 2)
    sc = A.read_path(np.ones((1, 2, d)), w["packed"], w["norms"], s, b)
    assert sc.shape == (1, 2, 0)


def test_score_condition_pins():
    """The tolerance scale ||k|| sum_j |q'_j c_idx_j|: a loop over every term
    (GQA head h reads KV head h // G), no smaller than |score| (triangle
    inequality), and equal to the score when every term is nonnegative."""
    keys, q, bits, b = _case(31, B=2, Hkv=2, G=2, T=5, d=32, b=3)
    s = A.signs_from_bits(bits)
    w = A.write_path(keys, s, b)
    c, _ = A.lloyd_max_codebook(32, b)
    qp = A.transform_queries(q, s)
    cond = A.score_condition(qp, w["idx"], w["norms"], c)
    B_, Hq, d = qp.shape
    G = Hq // w["idx"].shape[1]
    for bi in range(B_):
        for h in range(Hq):
            for t in range(w["idx"].shape[2]):
                kv = h // G
                terms = [abs(qp[bi, h, j] * c[w["idx"][bi, kv, t, j]]) for j in range(d)]
                assert cond[bi, h, t] == pytest.approx(w["norms"][bi, kv, t] * sum(terms),
                                                       rel=1e-13)
    score = A.read_path(q, w["packed"], w["norms"], s, b)
    assert np.all(np.abs(score) <= cond * (1 + 1e-13))
    # nonnegative terms: q' >= 0 and every index in the positive half
    idx_pos = np.full_like(w["idx"], (1 << b) - 1)
    qp_pos = np.abs(qp)
    lut = A.build_lut(qp_pos, c)
    direct = np.empty_like(cond)
    for bi in range(B_):
        for h in range(Hq):
            kv = h // G
            direct[bi, h] = w["norms"][bi, kv] * lut[bi, h][np.arange(d), idx_pos[bi, kv]].sum(-1)
    np.testing.assert_allclose(A.score_condition(qp_pos, idx_pos, w["norms"], c), direct,
                               rtol=1e-13)
    assert np.all(direct > 0)
