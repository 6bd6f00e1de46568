"""The oracle's pins must catch plausible mistakes.  Each test plants one
mistake in the oracle (on the CPU, via monkeypatch) and checks that the pin
that guards that step now fails."""

import math

import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import axelram as A
from tests._golden import max1960_table, pack_example
from tests.test_oracle_codebook import quadrature_centroid_residual
from tests.test_oracle_score import independent_dequantize_dot, _case
from tests.test_oracle_transform import butterfly_wht


def test_wrong_conditional_mean_is_caught(monkeypatch):
    # mistake: sign error in the conditional mean of a Gaussian cell
    orig = A.gaussian_cell_mean
    monkeypatch.setattr(A, "gaussian_cell_mean", lambda lo, hi: -orig(lo, hi) * 0.5)
    c, t = A.lloyd_max_codebook(128, 3, max_iter=500)
    assert not quadrature_centroid_residual(128, c, t) <= 1e-11


def test_codebook_for_wrong_variance_is_caught():
    # mistake: solve for N(0, 1) and forget the 1/sqrt(d) scale
    c, t = A.lloyd_max_codebook(1, 3)
    assert not quadrature_centroid_residual(128, c, t) <= 1e-11


def test_unscaled_table_is_caught():
    table = max1960_table()[3]
    c, _ = A.lloyd_max_codebook(4, 3)              # sigma = 1/2 instead of 1
    assert not np.allclose(c[4:], table["centroid"], rtol=6e-4, atol=6e-4)


def test_bit_reversed_hadamard_is_caught():
    d = 32
    rev = np.array([int(format(i, "05b")[::-1], 2) for i in range(d)])
    wrong = A.sylvester_hadamard(d)[rev]
    assert not np.array_equal(wrong, hadamard(d))


def test_signs_after_transform_is_caught(monkeypatch):
    d = 64
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, d))
    s = A.signs_from_bits(rng.integers(0, 2, d))
    h = A.sylvester_hadamard(d)
    monkeypatch.setattr(A, "rotate", lambda x_, s_: (np.asarray(x_) @ h.T) * s_ / math.sqrt(d))
    assert not np.allclose(A.rotate(x, s), butterfly_wht(s * x) / math.sqrt(d), atol=1e-13)


def test_missing_normalisation_is_caught(monkeypatch):
    d = 64
    rng = np.random.default_rng(2)
    s = A.signs_from_bits(rng.integers(0, 2, d))
    monkeypatch.setattr(A, "rotate", lambda x_, s_: butterfly_wht(np.asarray(x_) * s_))
    x = rng.standard_normal((4, d))
    y = A.rotate(x, s)
    assert not np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1))


def test_ties_going_up_is_caught(monkeypatch):
    monkeypatch.setattr(A, "quantize", lambda y, t: np.sum(np.asarray(y)[..., None] >= t, axis=-1))
    _, t = A.lloyd_max_codebook(128, 3)
    assert not np.array_equal(A.quantize(t, t), np.arange(len(t)))


def test_msb_first_fields_are_caught(monkeypatch):
    ex = pack_example()
    orig = A.pack_indices

    def msb_first(idx, b):
        idx = np.asarray(idx)
        rev = sum(((idx >> r) & 1) << (b - 1 - r) for r in range(b))
        return orig(rev, b)

    monkeypatch.setattr(A, "pack_indices", msb_first)
    words = A.pack_indices(np.arange(ex["d"]) % 8, ex["b"])
    assert [int(w) for w in words] != ex["words"]


def test_transposed_table_is_caught(monkeypatch):
    keys, q, bits, b = _case(31, d=32, b=3)
    s = A.signs_from_bits(bits)
    w = A.write_path(keys, s, b)
    c, _ = A.lloyd_max_codebook(32, b)
    ref = independent_dequantize_dot(q, w["idx"], w["norms"], bits, c)

    def wrong_gather(lut_h, idx_h):          # reads LUT[idx_j mod d', j mod 2^b]
        d = lut_h.shape[0]
        flat = lut_h.reshape(-1)
        return flat[(idx_h * d + np.arange(d)[None, :]) % flat.size]

    monkeypatch.setattr(A, "_gather", wrong_gather)
    got = A.lut_scores(A.transform_queries(q, s), w["idx"], w["norms"], c)
    assert not np.allclose(got, ref, rtol=1e-9, atol=1e-9)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    keys, q, bits, b = _case(32, Hkv=2, G=2, d=32)
    keys[:, 1] = 0.0
    s = A.signs_from_bits(bits)
    w = A.write_path(keys, s, b)
    c, _ = A.lloyd_max_codebook(32, b)

    def interleaved(qprime, idx, norms, centroids):   # mistake: kv = h % Hkv
        lut = A.build_lut(qprime, centroids)
        hkv = idx.shape[1]
        out = np.empty((qprime.shape[0], qprime.shape[1], idx.shape[2]))
        for bi in range(qprime.shape[0]):
            for h in range(qprime.shape[1]):
                out[bi, h] = norms[bi, h % hkv] * A._gather(lut[bi, h], idx[bi, h % hkv]).sum(-1)
        return out

    monkeypatch.setattr(A, "lut_scores", interleaved)
    sc = A.read_path(q, w["packed"], w["norms"], s, b)
    assert not np.all(sc[:, 2:] == 0.0)


def test_append_into_the_next_slot_is_caught(monkeypatch):
    # mistake: the new key lands one slot after its position
    from tests import test_oracle_decode as D
    orig = A.append_keys
    monkeypatch.setattr(A, "append_keys",
                        lambda p, n, k, pos, s, b: orig(p, n, k, np.asarray(pos) + 1, s, b))
    with pytest.raises(AssertionError):
        D.test_append_token_by_token_equals_bulk_write(3)


def test_ragged_length_off_by_one_is_caught(monkeypatch):
    # mistake: each row scores one token more than its length
    from tests import test_oracle_decode as D
    orig = A.read_path_ragged
    monkeypatch.setattr(A, "read_path_ragged",
                        lambda q, p, n, s, b, lens, T: orig(q, p, n, s, b, np.asarray(lens) + 1, T))
    with pytest.raises(AssertionError):
        D.test_read_path_ragged_is_read_path_on_each_prefix()


def test_softmax_without_max_shift_is_caught(monkeypatch):
    # mistake: exponentiate the raw scores (no max subtraction)
    from tests import test_oracle_softmax as S

    def naive(scores, lens, scale):
        s = np.asarray(scores, np.float64)
        p = np.full(s.shape, np.nan)
        lse = np.full(s.shape[:2], -np.inf)
        for bi, n in enumerate(np.asarray(lens).tolist()):
            n = min(max(int(n), 0), s.shape[2])
            if n:
                e = np.exp(scale * s[bi, :, :n])
                p[bi, :, :n] = e / e.sum(axis=-1, keepdims=True)
                lse[bi] = np.log(e.sum(axis=-1))
        return p, lse
    monkeypatch.setattr(A, "softmax_probs", naive)
    with np.errstate(over="ignore", invalid="ignore"):
        with pytest.raises(AssertionError):
            S.test_large_scores_do_not_overflow()


def test_softmax_over_the_whole_row_is_caught(monkeypatch):
    # mistake: normalise over all T tokens instead of the row's length
    from tests import test_oracle_softmax as S
    orig = A.softmax_probs
    monkeypatch.setattr(A, "softmax_probs",
                        lambda s_, lens, scale: orig(s_, np.full(len(lens), np.shape(s_)[2]),
                                                     scale))
    with pytest.raises(AssertionError):
        S.test_equals_scipy_on_each_prefix(1.0)


def test_absolute_selection_error_is_caught(monkeypatch):
    # mistake: rank candidates by absolute error, so the loudest layer decides
    from tests import test_oracle_signsel as P
    orig = A.sign_selection_errors

    def absolute(keys, q, cands, b):
        e = orig(keys, q, cands, b)
        e[..., 1] = 1.0
        return e
    monkeypatch.setattr(A, "sign_selection_errors", absolute)
    with pytest.raises(AssertionError):
        P.test_sample_scale_does_not_change_relative_error()


def test_selection_gqa_mapping_mistake_is_caught(monkeypatch):
    # mistake: query head h reads KV head h % Hkv
    from tests import test_oracle_signsel as P

    def wrong(q, keys):
        q = np.asarray(q, np.float64)
        k = np.asarray(keys, np.float64)
        out = np.empty((q.shape[0], q.shape[1], k.shape[2]))
        for bi in range(q.shape[0]):
            for h in range(q.shape[1]):
                out[bi, h] = k[bi, h % k.shape[1]] @ q[bi, h]
        return out
    monkeypatch.setattr(A, "dense_scores", wrong)
    with pytest.raises(AssertionError):
        P.test_dense_scores_gqa_mapping()


def test_hamilton_sign_error_is_caught(monkeypatch):
    # mistake: one cross term of the product with the wrong sign
    from tests import test_oracle_isoquant as Q

    def wrong(a, b):
        a = np.asarray(a, np.float64)
        b = np.asarray(b, np.float64)
        aw, ax, ay, az = a[..., 0], a[..., 1], a[..., 2], a[..., 3]
        bw, bx, by, bz = b[..., 0], b[..., 1], b[..., 2], b[..., 3]
        return np.stack([aw * bw - ax * bx - ay * by - az * bz,
                         aw * bx + ax * bw - ay * bz - az * by,
                         aw * by - ax * bz + ay * bw + az * bx,
                         aw * bz + ax * by - ay * bx + az * bw], axis=-1)
    monkeypatch.setattr(A, "quaternion_multiply", wrong)
    with pytest.raises(AssertionError):
        Q.test_hamilton_units()


def test_fast_rotation_on_the_wrong_side_is_caught(monkeypatch):
    # mistake: the Fast variant multiplies on the right (v q_L)
    from tests import test_oracle_isoquant as Q
    orig = A.isoquant_rotate

    def wrong(x, ql, qr=None):
        if qr is not None:
            return orig(x, ql, qr)
        x = np.asarray(x, np.float64)
        v = x.reshape(*x.shape[:-1], x.shape[-1] // 4, 4)
        return A.quaternion_multiply(v, np.asarray(ql, np.float64)).reshape(x.shape)
    monkeypatch.setattr(A, "isoquant_rotate", wrong)
    with pytest.raises(AssertionError):
        Q.test_rotation_preserves_norms_and_inverts(False)
