"""CPU checks of the parity helpers the GPU tests rely on: the softmax check
accepts fp32-rounded probabilities, rejects planted errors, and stays defined
when reference probabilities underflow fp64 (scores spread over thousands of
units after scaling)."""

import numpy as np
import pytest

from oracle import axelram as A
from tests._parity import assert_softmax


def _row(spread, T=64, seed=0):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal((2, T)) * spread
    cond = np.abs(ref) + 1.0
    return ref, cond


@pytest.mark.parametrize("spread", [1.0, 50.0, 1e4, 1e9])
def test_fp32_probabilities_pass(spread):
    ref, cond = _row(spread)
    p, lse = A.softmax_probs(ref[None], [ref.shape[1]], 1.0)
    assert_softmax(p[0].astype(np.float32), lse[0].astype(np.float32), ref, cond, 1.0,
                   ref.shape[1])


def test_underflowed_reference_probabilities_are_checked_in_log_domain():
    """Scaled scores 800 apart: the reference probability of the low token is
    exp(-800), 0 in fp64; a GPU value of 0 passes and one of 1e-30 does not
    (the bound on its log is a few units)."""
    ref = np.array([[0.0, -800.0, -1.0]])
    cond = np.full_like(ref, 1e-3)
    p, lse = A.softmax_probs(ref[None], [3], 1.0)
    got = p[0].copy()
    assert got[0, 1] == 0.0
    assert_softmax(got, lse[0], ref, cond, 1.0, 3)
    got[0, 1] = 1e-30
    with pytest.raises(AssertionError):
        assert_softmax(got, lse[0], ref, cond, 1.0, 3)


def test_planted_probability_error_fails():
    ref, cond = _row(3.0)
    cond = cond * 1e-6                       # a tight score tolerance
    p, lse = A.softmax_probs(ref[None], [ref.shape[1]], 1.0)
    got = p[0].copy()
    got[1, 5] *= 1.01
    with pytest.raises(AssertionError):
        assert_softmax(got, lse[0], ref, cond, 1.0, ref.shape[1])


def test_index_mismatch_cap():
    """In-window flips: two are allowed on a small array, a third fails; one
    outside the window always fails."""
    from tests._parity import assert_indices
    t = np.array([-0.5, 0.0, 0.5])
    y = np.linspace(-1.0, 1.0, 1000)
    y[[10, 20, 30]] = [0.5 + 1e-7, -0.5 - 2e-7, 3e-7]
    ora = A.quantize(y, t)
    got = ora.copy()
    got[[10, 20]] += np.array([-1, 1])
    assert assert_indices(got, ora, y, t)[0] == 2
    got[30] -= 1
    with pytest.raises(AssertionError):
        assert_indices(got, ora, y, t)
    far = ora.copy()
    far[500] += 1
    with pytest.raises(AssertionError):
        assert_indices(far, ora, y, t)
