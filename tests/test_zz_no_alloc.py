"""axr_score_softmax_noalloc (split-T partials in the library's own device
array, for callers that cannot allocate) against axr_score_softmax with a
caller workspace and against the oracle, on two calls in a row, the second
with a smaller input (the array still holds the first call's partials, which
the second must not read).

The two entry points run the same kernels, but the score kernel hands token
units to its waves dynamically, so the order in which a tile's exponentials
are summed (and the last bit of each row's sum) differs from launch to
launch: probabilities and log-sum-exps are compared to a relative 1e-5
(three orders above that rounding, far below any mixed-up partial), and both
meet the oracle's softmax bound."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, assert_softmax

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
AGREE_RTOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lut_attention_scoring_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _case(B, Hkv, G, T, d, b, seed, ragged):
    import lut_attention_scoring_amd as m
    rng = np.random.default_rng(seed)
    keys = torch.from_numpy((rng.standard_normal((B, Hkv, T, d)) * 2.0).astype(np.float32)
                            ).to(torch.float16)
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32))
    bits = W.sign_bits(d)
    packed, norms = m.quantize_keys(keys.to(DEV), bits, b)
    lens = None
    if ragged:
        lens = torch.from_numpy(rng.integers(0, T + 3, size=B).astype(np.int32)).to(DEV)
    return keys, q, packed, norms, bits, lens


def _oracle_check(keys, q, packed, bits, b, probs, lse, lens, label):
    d = q.shape[-1]
    T = keys.shape[2]
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(q), s)
    got, glse = f64(probs), f64(lse)
    n = lens.cpu().numpy().clip(0, T) if lens is not None else np.full(q.shape[0], T)
    for bi in range(q.shape[0]):
        if n[bi] == 0:
            assert np.all(np.isneginf(glse[bi])), label
            continue
        gidx = A.unpack_indices(words_u32(packed[bi:bi + 1, :, :n[bi]]), d, b)
        onorm = A.key_norms(f64(keys[bi:bi + 1, :, :n[bi]]))
        ref = A.lut_scores(qprime[bi:bi + 1], gidx, onorm, c)[0]
        cond = A.score_condition(qprime[bi:bi + 1], gidx, onorm, c)[0]
        assert_softmax(got[bi], glse[bi], ref, cond, 1.0 / np.sqrt(d), int(n[bi]),
                       f"{label} bi={bi}")


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    import lut_attention_scoring_amd as m
    big = dict(B=8, Hkv=8, G=4, T=6000, d=128, b=3, seed=1, ragged=True)
    small = dict(B=1, Hkv=2, G=8, T=700, d=256, b=4, seed=2, ragged=False)
    seq = [big, small] if order == "large_then_small" else [small, big, small]
    for k, cfg in enumerate(seq):
        label = f"no-alloc call {k}: {cfg}"
        print(label, flush=True)
        keys, q, packed, norms, bits, lens = _case(**cfg)
        qd = q.to(DEV)
        B, Hq, T = q.shape[0], q.shape[1], cfg["T"]
        p_ws, l_ws = m.score_softmax(qd, packed, norms, bits, cfg["b"], lens=lens)
        out = torch.full((B, Hq, T), float("nan"), device=DEV)
        lse = torch.full((B, Hq), float("nan"), device=DEV)
        p_na, l_na = m.score_softmax_noalloc(qd, packed, norms, bits, cfg["b"], out=out, lse=lse,
                                             lens=lens)
        torch.cuda.synchronize()
        n = lens.cpu().numpy().clip(0, T) if lens is not None else np.full(B, T)
        lw, ln = f64(l_ws), f64(l_na)
        fin = np.isfinite(lw)
        assert np.array_equal(fin, np.isfinite(ln)), label
        assert np.all(lw[~fin] == ln[~fin]), label
        assert np.all(np.abs(lw[fin] - ln[fin]) <= AGREE_RTOL * (1.0 + np.abs(lw[fin]))), label
        for bi in range(B):
            a, z = f64(p_ws[bi, :, :n[bi]]), f64(p_na[bi, :, :n[bi]])
            assert np.all(np.abs(a - z) <= AGREE_RTOL * a + 2.0 ** -126), label
            assert torch.isnan(p_na[bi, :, n[bi]:]).all(), f"{label}: wrote past the row"
        _oracle_check(keys, q, packed, bits, cfg["b"], p_na, l_na, lens, label)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """B * Hq * tiles * 8 bytes of partials over the library's 1 MiB: rejected
    before any device work, nothing written."""
    import lut_attention_scoring_amd as m
    B, Hkv, G, T, d, b = 4096, 1, 64, 1, 128, 3
    q = torch.zeros(B, Hkv * G, d, dtype=torch.float16, device=DEV)
    packed = torch.zeros(B, Hkv, T, d * b // 32, dtype=torch.int32, device=DEV)
    norms = torch.zeros(B, Hkv, T, device=DEV)
    out = torch.full((B, Hkv * G, T), 7.0, device=DEV)
    lse = torch.full((B, Hkv * G), 7.0, device=DEV)
    with pytest.raises(m.AxrError) as ei:
        m.score_softmax_noalloc(q, packed, norms, W.sign_bits(d), b, out=out, lse=lse)
    assert ei.value.status == m.EUNSUPPORTED and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert (out == 7.0).all() and (lse == 7.0).all()
