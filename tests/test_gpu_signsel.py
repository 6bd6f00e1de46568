"""GPU parity of the one-time sign-pattern selection (AXELRAM, Abstract:
gradient-free selection among candidate sign patterns on calibration
samples; scored here by the table scores' distance from the exact scores).

The GPU's per-(candidate, sample) sums are compared with the oracle's sums
built from the GPU's own indices (the same write kernel, called per
candidate) and exact fp64 scores.  Bound per score: the table score is within
1e-5 of its condition scale, the fp32 exact score within d * 2^-24 of
sum_j |q_j k_j| plus its rounding; the bound on the sums follows from
|(D + e)^2 - D^2| <= 2 |D| e + e^2."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, SCORE_RTOL

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lut_attention_scoring_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def axr():
    import lut_attention_scoring_amd as m
    return m


def _oracle_sums(keys_s, q_s, gpu_packed, bits, b):
    """err, ref and their bounds for one sample from the GPU's records."""
    d = keys_s.shape[-1]
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    k64, q64 = f64(keys_s), f64(q_s)
    gidx = A.unpack_indices(words_u32(gpu_packed), d, b)
    onorm = A.key_norms(k64)
    qprime = A.transform_queries(q64, s)
    lut = A.lut_scores(qprime, gidx, onorm, c)
    cond = A.score_condition(qprime, gidx, onorm, c)
    exact = A.dense_scores(q64, k64)
    G = q64.shape[1] // k64.shape[1]
    absdot = np.einsum("bhd,bhtd->bht", np.abs(q64), np.repeat(np.abs(k64), G, axis=1))
    delta = lut - exact
    eps = SCORE_RTOL * cond + d * 2.0 ** -24 * absdot + 2.0 ** -23 * np.abs(exact)
    err, ref = np.sum(delta ** 2), np.sum(exact ** 2)
    err_bound = np.sum(2 * np.abs(delta) * eps + eps ** 2) + 1e-12 * err
    ref_bound = np.sum(2 * np.abs(exact) * (d * 2.0 ** -24 * absdot + 2.0 ** -23 * np.abs(exact))
                       ) + 1e-12 * ref
    return err, ref, err_bound, ref_bound


def _check(keys, q, cand_bits, b, which, label):
    m = axr()
    e = m.sign_selection_errors(keys.to(DEV), q.to(DEV), cand_bits, b).cpu().numpy()
    S = keys.shape[0]
    for ci in which:
        packed, _ = m.quantize_keys(keys.to(DEV), cand_bits[ci], b)
        torch.cuda.synchronize()
        for i in range(S):
            err, ref, eb, rb = _oracle_sums(keys[i], q[i], packed[i], cand_bits[ci], b)
            assert abs(e[ci, i, 1] - ref) <= rb, f"{label} c={ci} i={i}: ref"
            assert abs(e[ci, i, 0] - err) <= eb, \
                f"{label} c={ci} i={i}: err {e[ci, i, 0]:.6e} vs {err:.6e} (bound {eb:.2e})"
    return e


@pytest.mark.parametrize("b", [2, 3, 4])
def test_selection_errors_small(b):
    cal = W.calibration_samples(count=3, T=300, seed=200 + b)
    rng = np.random.default_rng(b)
    bits = rng.integers(0, 2, size=(3, 128)).astype(np.uint8)
    cands = np.concatenate([bits, 1 - bits[:1]])            # candidate 3 negates candidate 0
    e = _check(cal["keys"], cal["q"], cands, b, range(len(cands)), f"b={b}")
    # a negated pattern mirrors every index: same sums up to the same bounds
    r0 = e[0, :, 0] / e[0, :, 1]
    r3 = e[3, :, 0] / e[3, :, 1]
    assert np.allclose(r0, r3, rtol=1e-3)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_selection_errors_dtypes_and_gqa(dtype):
    rng = np.random.default_rng(17)
    keys = torch.from_numpy((rng.standard_normal((2, 2, 1, 257, 256)) + 0.5).astype(np.float32)
                            ).to(dtype)
    q = torch.from_numpy(rng.standard_normal((2, 2, 4, 256)).astype(np.float32)).to(dtype)
    cands = rng.integers(0, 2, size=(2, 256)).astype(np.uint8)
    _check(keys, q, cands, 3, range(2), f"{dtype}")


def test_selection_full_calibration_set():
    """200 candidates on 8 calibration layers (B=1, 2 KV heads, 16 query heads,
    2048 tokens, d=128, b=4): sums checked against the oracle for the default
    pattern, the chosen one and the worst one; the choice is the argmin."""
    m = axr()
    cal = W.calibration_samples()
    cands = W.sign_candidates(128)
    keys, q = cal["keys"].to(DEV), cal["q"].to(DEV)
    idx, objective = m.select_sign_pattern(keys, q, cands, 4)
    assert objective.shape == (len(cands),) and np.all(np.isfinite(objective))
    # the library's choice equals the oracle's rule applied to the GPU's sums
    e = m.sign_selection_errors(keys, q, cands, 4).cpu().numpy()
    oidx, oobj = A.select_sign_pattern(e)
    assert idx == oidx and np.array_equal(objective, oobj)
    worst = int(np.argmax(objective))
    _check(cal["keys"], cal["q"], cands, 4, sorted({0, idx, worst}), "full")


@pytest.mark.parametrize("i", range(8))
def test_selection_errors_random_shapes(i):
    """Seeded random shapes of the selection inputs: samples, batch, KV heads,
    group size, tokens, d, b, dtypes; every candidate's sums against the
    oracle's from the GPU's own indices."""
    rng = np.random.default_rng(9500 + i)
    S = int(rng.integers(1, 4))
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    T = int(rng.integers(1, 900))
    d = int(rng.choice([128, 256]))
    b = int(rng.integers(2, 5))
    dtype = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))]
    C = int(rng.integers(1, 4))
    label = f"selection random {i}: S={S} B={B} Hkv={Hkv} G={G} T={T} d={d} b={b} {dtype} C={C}"
    print(label, flush=True)
    keys = torch.from_numpy((rng.standard_normal((S, B, Hkv, T, d)) * np.exp(
        rng.standard_normal(d)) + 0.3).astype(np.float32)).to(dtype)
    q = torch.from_numpy(rng.standard_normal((S, B, Hkv * G, d)).astype(np.float32)).to(dtype)
    cands = rng.integers(0, 2, size=(C, d)).astype(np.uint8)
    e = _check(keys, q, cands, b, range(C), label)
    idx, obj = axr().sign_selection_choose(e)
    oidx, oobj = A.select_sign_pattern(e)
    assert idx == oidx and np.array_equal(obj, oobj), label


def test_selection_with_a_zero_query_sample():
    """A calibration sample whose queries are all zero has no exact score
    mass (ref = 0) and zero table scores (err = 0): it counts 0 and the
    choice is made by the other samples, as the oracle's rule says."""
    m = axr()
    cal = W.calibration_samples(count=3, T=256, seed=301)
    q = cal["q"].clone()
    q[1] = 0
    cands = W.sign_candidates(128, count=6)
    e = m.sign_selection_errors(cal["keys"].to(DEV), q.to(DEV), cands, 3).cpu().numpy()
    assert np.all(e[:, 1, :] == 0.0)
    idx, obj = m.sign_selection_choose(e)
    oidx, oobj = A.select_sign_pattern(e)
    assert idx == oidx and np.array_equal(obj, oobj) and np.all(np.isfinite(obj))
