"""The score kernel's fixed-point table, emulated on the CPU.

The read path (AXELRAM, Abstract: each key's score is its norm times the sum
of the table entries its indices select) is summed on the GPU in 32-bit
integers: per query head a power of two 2^sh is chosen with
sum_j |q'_j| max|c| 2^sh < 2^31 (with a 1.0001 guard factor), every
coordinate term q'_j c_k 2^sh is rounded to an integer, and the integer sum
is scaled back by 2^-sh and multiplied by the key's norm in fp32.  This test
models those steps in numpy (fp32 products, round-half-even, exact integer
sums) on the worst-case inputs of tests/_adversarial.py and checks:

* the error stays within the derived bound d/2 * 1.0001 * (max|c| / min|c|)
  / 2^30 of ||k|| sum_j |LUT[j][idx_j]| (plus a few fp32 roundings), which is
  at most 5.1e-6 (d = 512, b = 4): half the 1e-5 parity bound;
* the inputs are really the worst case: they reach 90 % of that bound, and
  with the full scale one bit lower (2^30) they come within 10 % of 1e-5;
* the integer sums fit int32 for every index pattern.

It models the kernel's design; it is not the oracle (the exact scores come
from oracle.axelram).  At d = 128, b = 4 the kernel keeps fp32 entries
instead (the signed half table of 4-bit pairs, summed in fp32); there the
integer model below is a bound of a design not in use, and the kernel's own
arithmetic is checked on the GPU (tests/test_gpu_score_bound.py)."""

import numpy as np
import pytest

from oracle import axelram as A
from tests import _adversarial as ADV

FP32_SLACK = 6 * 2.0 ** -24      # q', products, int->float, norm, final multiply


def _kernel_model(q, idx, norms, d, b, signs, top_bit=31):
    """Scores [G, T] of queries q [G, d] against indices idx [T, d] and norms
    [T], with the kernel's arithmetic; also returns the integer sums."""
    c, _ = ADV.codebook(d, b)
    cf = c.astype(np.float32)
    # q' in fp32: the one-hot transform is exact up to the final 1/sqrt(d)
    qf = A.transform_queries(q[None], signs)[0].astype(np.float32)
    out = np.empty((q.shape[0], idx.shape[0]))
    sums = np.empty_like(out, dtype=np.int64)
    for g in range(q.shape[0]):
        sa = np.float32(0.0)
        for v in np.abs(qf[g]):
            sa = np.float32(sa + v)
        f = np.float32(np.float32(sa * cf[-1]) * np.float32(ADV.SCALE_GUARD))
        _, e = np.frexp(f)                           # f < 2^e
        sh = top_bit - int(e)
        qa = (qf[g] * np.float32(2.0 ** sh)).astype(np.float32)   # exact
        terms = np.rint((qa[None, :] * cf[idx]).astype(np.float32)).astype(np.int64)
        tot = terms.sum(axis=1)
        sums[g] = tot
        inv = np.float32(2.0 ** -sh)
        out[g] = (norms.astype(np.float32) * (tot.astype(np.float32) * inv)).astype(np.float32)
    return out, sums


def _errors(d, b, top_bit, G=16, T=96, seed=0):
    q, k, bits = ADV.worst_case_inputs(d, b, G, T, seed)
    s = A.signs_from_bits(bits)
    _, t = ADV.codebook(d, b)
    c, _ = ADV.codebook(d, b)
    y, norms = A.transform_keys(k[0, 0], s)
    idx = A.quantize(y, t)
    got, sums = _kernel_model(q[0], idx, norms, d, b, s, top_bit)
    qp = A.transform_queries(q, s)
    ref = A.lut_scores(qp, idx[None, None], norms[None, None], c)[0]
    cond = A.score_condition(qp, idx[None, None], norms[None, None], c)[0]
    return np.abs(got - ref) / cond, sums


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_worst_case_within_derived_bound(d, b):
    rel, sums = _errors(d, b, 31)
    bound = ADV.table_rounding_bound(d, b)
    assert rel.max() <= bound + FP32_SLACK, (rel.max(), bound)
    assert rel.max() <= 0.55e-5
    assert np.abs(sums).max() < 2 ** 31


def test_inputs_reach_the_bound():
    """At d = 512, b = 4 the constructed inputs come within 10 % of the
    derived bound, and a full scale one bit lower (2^30) would leave under
    10 % of the 1e-5 parity bound as margin."""
    rel, _ = _errors(512, 4, 31)
    assert rel.max() >= 0.9 * ADV.table_rounding_bound(512, 4)
    rel30, _ = _errors(512, 4, 30)
    assert rel30.max() >= 0.9e-5


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 512])
def test_integer_sums_fit_int32_for_any_indices(d, b):
    """Every index in the top or bottom cell, signed to add up (the largest
    possible |sum|), for flat and spiky query transforms."""
    rng = np.random.default_rng(d + b)
    c, _ = ADV.codebook(d, b)
    s = np.ones(d)
    q = np.vstack([ADV.one_hot_queries(d, b, 4, rng), rng.standard_normal((4, d))])
    qp = A.transform_queries(q[None], s)[0]
    idx = np.where(qp >= 0, len(c) - 1, 0)          # every term positive and largest
    for g in range(q.shape[0]):
        _, sums = _kernel_model(q[g:g + 1], idx[g:g + 1], np.ones(1), d, b, s)
        assert 2 ** 30 * 0.999 <= abs(int(sums[0, 0])) < 2 ** 31
