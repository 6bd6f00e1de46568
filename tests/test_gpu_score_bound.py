"""GPU parity on the worst case of the score kernel's fixed-point table.

The inputs of tests/_adversarial.py (one-hot queries whose full scale sits at
the bottom of its range, unit keys with every transformed coordinate but one
at the smallest positive centroid, signed so that every term of a score is
positive) make the table's roundings add up.  The kernel's scores must stay
within the 1e-5 parity bound of ||k|| sum_j |LUT[j][idx_j]| and, more
tightly, within the derived table bound d/2 * 1.0001 * (max|c| / min|c|) /
2^30 plus 1e-6 for the fp32 norm and products (5.1e-6 + 1e-6 at d = 512,
b = 4), in the plain, softmax and fused decode-step launches."""

import numpy as np
import pytest
import torch

from oracle import axelram as A
from tests import _adversarial as ADV
from tests._parity import f64, words_u32, assert_scores, assert_softmax
from tests.test_gpu_parity import _write_and_check, _score_and_check

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FP32_SLACK = 1e-6

# (128, 2) runs the 4-coordinate table (8-bit fields), (128, 4) the signed
# half table, the others the int32 pair or single-coordinate tables.
CASES = [(512, 4), (256, 4), (512, 3), (128, 4), (128, 3), (128, 2)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lut_attention_scoring_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def axr():
    import lut_attention_scoring_amd as m
    return m


def _inputs(d, b, G=16, T=777, seed=0, powers=(0, -7, 9, 40)):
    q, k, bits = ADV.worst_case_inputs(d, b, G, T, seed=seed + d + b, powers=powers)
    return (torch.from_numpy(q.astype(np.float32)), torch.from_numpy(k.astype(np.float32)),
            bits)


def _oracle_ref(q_cpu, keys_cpu, packed, bits, b):
    d = q_cpu.shape[-1]
    s = A.signs_from_bits(bits)
    c, _ = ADV.codebook(d, b)
    qp = A.transform_queries(f64(q_cpu), s)
    gidx = A.unpack_indices(words_u32(packed), d, b)
    onorm = A.key_norms(f64(keys_cpu))
    return (A.lut_scores(qp, gidx, onorm, c), A.score_condition(qp, gidx, onorm, c), qp, gidx,
            onorm)


@pytest.mark.parametrize("d,b", CASES)
def test_worst_case_scores(d, b):
    q, keys, bits = _inputs(d, b)
    label = f"worst case d={d} b={b}"
    print(label, flush=True)
    packed, norms = _write_and_check(keys, bits, b, label)
    worst = _score_and_check(q, keys, packed, norms, bits, b, label)
    assert worst <= ADV.table_rounding_bound(d, b) + FP32_SLACK, (label, worst)


@pytest.mark.parametrize("d,b", CASES[:3])
@pytest.mark.parametrize("scale", [None, 400.0])
def test_worst_case_softmax(d, b, scale):
    m = axr()
    q, keys, bits = _inputs(d, b, seed=11)
    label = f"worst case softmax d={d} b={b} scale={scale}"
    print(label, flush=True)
    packed, norms = m.quantize_keys(keys.to(DEV), bits, b)
    probs, lse = m.score_softmax(q.to(DEV), packed, norms, bits, b, scale=scale)
    torch.cuda.synchronize()
    ref, cond, *_ = _oracle_ref(q, keys, packed.cpu(), bits, b)
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    T = keys.shape[2]
    assert_softmax(f64(probs[0]), f64(lse[0]), ref[0], cond[0], sc, T, label)


@pytest.mark.parametrize("d,b", CASES[:3])
def test_worst_case_fused_decode(d, b):
    """The last token is appended by the fused decode step (its record comes
    from the kernel's own quantization of the new key) and every token is
    scored with it in place."""
    m = axr()
    q, keys, bits = _inputs(d, b, seed=23)
    label = f"worst case decode d={d} b={b}"
    print(label, flush=True)
    T = keys.shape[2]
    packed, norms = m.quantize_keys(keys[:, :, :T - 1].to(DEV), bits, b)
    W = packed.shape[-1]
    cache = torch.zeros(1, 1, T, W, dtype=torch.int32, device=DEV)
    cnorm = torch.zeros(1, 1, T, dtype=torch.float32, device=DEV)
    cache[:, :, :T - 1] = packed
    cnorm[:, :, :T - 1] = norms
    pos = torch.full((1,), T - 1, dtype=torch.int32, device=DEV)
    scores = m.decode_step(q.to(DEV), keys[:, :, T - 1].contiguous().to(DEV), bits, b, cache,
                           cnorm, pos)
    torch.cuda.synchronize()
    ref, cond, qp, gidx, onorm = _oracle_ref(q, keys, cache.cpu(), bits, b)
    # the appended record against the oracle's quantization of the new key
    s = A.signs_from_bits(bits)
    _, t = ADV.codebook(d, b)
    y, _ = A.transform_keys(f64(keys[0, 0, T - 1:]), s)
    bad = gidx[0, 0, T - 1] != A.quantize(y, t)[0]
    if bad.any():
        dist = np.min(np.abs(y[0][bad][:, None] - t[None, :]), axis=1)
        assert dist.max() < 1e-6, label
    worst = assert_scores(f64(scores), qp, gidx, onorm, ADV.codebook(d, b)[0], label)
    assert worst <= ADV.table_rounding_bound(d, b) + FP32_SLACK, (label, worst)


@pytest.mark.parametrize("d,b", [(128, 3), (128, 2)])
def test_worst_case_quantize_score(d, b):
    """The one-launch write and read path on the same worst case (G = 4, one
    table per row): its scores against the derived table bound, its records
    against the oracle's quantization."""
    m = axr()
    q, keys, bits = _inputs(d, b, G=4, seed=31)
    label = f"worst case quantize-and-score d={d} b={b}"
    print(label, flush=True)
    packed, norms, scores = m.quantize_score(keys.to(DEV), q.to(DEV), bits, b)
    torch.cuda.synchronize()
    ref, cond, qp, gidx, onorm = _oracle_ref(q, keys, packed.cpu(), bits, b)
    s = A.signs_from_bits(bits)
    _, t = ADV.codebook(d, b)
    y, _ = A.transform_keys(f64(keys[0, 0]), s)
    bad = gidx[0, 0] != A.quantize(y, t)
    if bad.any():
        dist = np.min(np.abs(y[bad][:, None] - t[None, :]), axis=1)
        assert dist.max() < 1e-6, label
    worst = assert_scores(f64(scores), qp, gidx, onorm, ADV.codebook(d, b)[0], label)
    assert worst <= ADV.table_rounding_bound(d, b) + FP32_SLACK, (label, worst)
