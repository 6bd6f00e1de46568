"""Pins for the oracle's scalar quantizer and packed index record."""

import math

import numpy as np
import pytest

from oracle import axelram as A
from tests._golden import pack_example


def brute_force_nearest(y, centroids):
    """argmin_c |y - c|, first minimum on ties."""
    dist = np.abs(np.asarray(y)[..., None] - np.asarray(centroids))
    return np.argmin(dist, axis=-1)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [32, 128, 512])
def test_quantizer_is_nearest_codeword(b, d):
    c, t = A.lloyd_max_codebook(d, b)
    rng = np.random.default_rng(b * 1000 + d)
    y = rng.standard_normal(200000) / math.sqrt(d) * 1.5
    far = np.min(np.abs(y[:, None] - t[None, :]), axis=1) > 1e-12
    idx = A.quantize(y, t)
    np.testing.assert_array_equal(idx[far], brute_force_nearest(y[far], c))
    np.testing.assert_array_equal(idx, np.searchsorted(t, y, side="left"))


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_ties_take_the_lower_cell(b):
    c, t = A.lloyd_max_codebook(128, b)
    np.testing.assert_array_equal(A.quantize(t, t), np.arange(len(t)))
    # 0 is the middle threshold: an exactly zero coordinate gets 2^(b-1) - 1
    assert A.quantize(np.array([0.0]), t)[0] == 2 ** (b - 1) - 1
    assert A.quantize(np.array([-1e9]), t)[0] == 0
    assert A.quantize(np.array([1e9]), t)[0] == 2 ** b - 1


def test_pack_hand_example():
    ex = pack_example()
    idx = np.arange(ex["d"]) % 8
    words = A.pack_indices(idx, ex["b"])
    assert [int(w) for w in words] == ex["words"]


def bigint_pack(idx, b):
    acc = 0
    for j, v in enumerate(idx):
        acc |= int(v) << (j * b)
    n = len(idx) * b // 32
    return [(acc >> (32 * w)) & 0xFFFFFFFF for w in range(n)]


@pytest.mark.parametrize("b", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [32, 64, 128, 256, 512])
def test_pack_matches_bigint_and_roundtrips(b, d):
    rng = np.random.default_rng(d + b)
    idx = rng.integers(0, 2 ** b, size=(3, 5, d))
    words = A.pack_indices(idx, b)
    assert words.dtype == np.uint32 and words.shape == (3, 5, d * b // 32)
    for i in range(3):
        for j in range(5):
            assert [int(w) for w in words[i, j]] == bigint_pack(idx[i, j], b)
    np.testing.assert_array_equal(A.unpack_indices(words, d, b), idx)
