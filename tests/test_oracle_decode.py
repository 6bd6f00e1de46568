"""Pins of the oracle's decode-step functions to the pinned write and read
paths ("AXELRAM: Quantize Once, Never Dequantize", Abstract: each key is
quantized once, when it is written, and scored by table lookup).

* A cache built one token at a time with append_keys equals write_path over
  all tokens at once: appending is the write path applied to one key.
* Slots outside [0, t_cap) and every other slot are left untouched.
* read_path_ragged equals read_path on each row's own prefix of tokens.
"""

import numpy as np
import pytest

from oracle import axelram as A
import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _cache(B, Hkv, T, d, b, seed):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((B, Hkv, T, d))
    s = A.signs_from_bits(W.sign_bits(d))
    return keys, s, A.write_path(keys, s, b)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_append_token_by_token_equals_bulk_write(b):
    B, Hkv, T, d = 2, 2, 9, 32
    keys, s, bulk = _cache(B, Hkv, T, d, b, seed=11)
    W_ = d * b // 32
    packed = np.zeros((B, Hkv, T, W_), dtype=np.uint32)
    norms = np.zeros((B, Hkv, T))
    for t in range(T):
        pos = np.full(B, t, dtype=np.int32)
        packed, norms = A.append_keys(packed, norms, keys[:, :, t], pos, s, b)
    assert np.array_equal(packed, bulk["packed"])
    assert np.array_equal(norms, bulk["norms"])


def test_append_ragged_slots_and_out_of_range():
    B, Hkv, T, d, b = 4, 3, 6, 32, 3
    keys, s, bulk = _cache(B, Hkv, T, d, b, seed=12)
    new = np.random.default_rng(13).standard_normal((B, Hkv, d))
    pos = np.array([0, 5, -1, 6], dtype=np.int32)       # last two are outside [0, 6)
    p2, n2 = A.append_keys(bulk["packed"], bulk["norms"], new, pos, s, b)
    one = A.write_path(new, s, b)
    for bi in range(B):
        for t in range(T):
            if t == pos[bi]:
                assert np.array_equal(p2[bi, :, t], one["packed"][bi])
                assert np.array_equal(n2[bi, :, t], one["norms"][bi])
            else:
                assert np.array_equal(p2[bi, :, t], bulk["packed"][bi, :, t])
                assert np.array_equal(n2[bi, :, t], bulk["norms"][bi, :, t])
    # inputs are not modified
    assert np.array_equal(bulk["packed"], A.write_path(keys, s, b)["packed"])


def test_read_path_ragged_is_read_path_on_each_prefix():
    B, Hkv, Hq, T, d, b = 3, 2, 4, 10, 32, 3
    keys, s, bulk = _cache(B, Hkv, T, d, b, seed=14)
    q = np.random.default_rng(15).standard_normal((B, Hq, d))
    lens = np.array([0, 7, 25], dtype=np.int32)        # empty, partial, longer than T
    got = A.read_path_ragged(q, bulk["packed"], bulk["norms"], s, b, lens, T)
    for bi in range(B):
        n_tok = min(max(int(lens[bi]), 0), T)
        assert np.all(np.isnan(got[bi, :, n_tok:]))
        if n_tok:
            ref = A.read_path(q[bi:bi + 1], bulk["packed"][bi:bi + 1, :, :n_tok],
                              bulk["norms"][bi:bi + 1, :, :n_tok], s, b)
            assert np.array_equal(got[bi, :, :n_tok], ref[0])
    full = A.read_path_ragged(q, bulk["packed"], bulk["norms"], s, b, np.full(B, T), T)
    assert np.array_equal(full, A.read_path(q, bulk["packed"], bulk["norms"], s, b))


def test_read_path_ragged_negative_length_scores_nothing():
    B, Hkv, Hq, T, d, b = 1, 1, 2, 4, 32, 2
    keys, s, bulk = _cache(B, Hkv, T, d, b, seed=16)
    q = np.ones((B, Hq, d))
    got = A.read_path_ragged(q, bulk["packed"], bulk["norms"], s, b, np.array([-3]), T)
    assert np.all(np.isnan(got))
