"""GPU parity of attention probabilities over the table-lookup scores
(axr_score_softmax): the split-T partials and the row normalisation against
the oracle's softmax of the exact scores of the GPU's own indices, within the
bound derived from the score tolerance and fp32 rounding (tests/_parity.py)."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, assert_softmax

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = 12345.5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lut_attention_scoring_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def axr():
    import lut_attention_scoring_amd as m
    return m


def _run(d, b, G, lens, T, t_cap, scale, key_scale=2.0, seed=0, Hkv=2, dtype=torch.float16):
    m = axr()
    rng = np.random.default_rng(seed)
    B = len(lens)
    bits = W.sign_bits(d)
    keys = torch.from_numpy((rng.standard_normal((B, Hkv, t_cap, d)) * key_scale).astype(
        np.float32)).to(dtype)
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32)).to(dtype)
    packed, norms = m.quantize_keys(keys.to(DEV), bits, b)
    out = torch.full((B, Hkv * G, T), SENTINEL, device=DEV)
    lse = torch.full((B, Hkv * G), SENTINEL, device=DEV)
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    m.score_softmax(q.to(DEV), packed, norms, bits, b, scale=scale, T=T, lens=lt, out=out,
                    lse=lse)
    torch.cuda.synchronize()
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(q), s)
    got, glse = f64(out), f64(lse)
    for bi, length in enumerate(lens):
        n_tok = min(max(length, 0), T)
        assert np.all(got[bi, :, n_tok:] == SENTINEL), f"bi={bi} wrote past its length"
        if n_tok == 0:
            assert np.all(np.isneginf(glse[bi])), f"bi={bi}: empty row lse"
            continue
        gidx = A.unpack_indices(words_u32(packed[bi:bi + 1, :, :n_tok]), d, b)
        onorm = A.key_norms(f64(keys[bi:bi + 1, :, :n_tok]))
        ref = A.lut_scores(qprime[bi:bi + 1], gidx, onorm, c)[0]
        cond = A.score_condition(qprime[bi:bi + 1], gidx, onorm, c)[0]
        assert_softmax(got[bi], glse[bi], ref, cond, scale, n_tok, f"bi={bi} len={n_tok}")


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("b", [2, 3, 4])
def test_softmax_ragged(G, b):
    _run(128, b, G, [0, 1, 300, 5000, 9000, -2, 4097, 2049], T=5000, t_cap=5200,
         scale=1.0 / math.sqrt(128), seed=10 * G + b)


@pytest.mark.parametrize("d,G", [(256, 4), (256, 8), (512, 4), (512, 8)])
def test_softmax_wide_heads(d, G):
    _run(d, 3, G, [1, 777, 3000], T=3000, t_cap=3000, scale=1.0 / math.sqrt(d), seed=d + G)


def test_softmax_large_scores_need_the_max_shift():
    # scores in the hundreds with scale 1: exp(scale * s) overflows fp32
    _run(128, 3, 4, [2000, 64, 1], T=2000, t_cap=2048, scale=1.0, key_scale=40.0, seed=5,
         dtype=torch.float32)


def test_softmax_full_lengths_match_dense_scores_row_sums():
    m = axr()
    rng = np.random.default_rng(9)
    d, b, B, Hkv, G, T = 128, 3, 2, 2, 4, 4096
    bits = W.sign_bits(d)
    keys = torch.from_numpy(rng.standard_normal((B, Hkv, T, d)).astype(np.float32)).to(DEV)
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32)).to(DEV)
    packed, norms = m.quantize_keys(keys, bits, b)
    probs, lse = m.score_softmax(q, packed, norms, bits, b)
    scores = m.score(q, packed, norms, bits, b)
    torch.cuda.synchronize()
    sc = f64(scores) / math.sqrt(d)
    ref_lse = np.log(np.exp(sc - sc.max(-1, keepdims=True)).sum(-1)) + sc.max(-1)
    assert np.allclose(f64(lse), ref_lse, rtol=0, atol=2e-5)
    assert np.allclose(f64(probs).sum(-1), 1.0, atol=2e-5)


def test_softmax_llama_full_size_sampled_rows():
    """The LLaMA-3.1-8B-shaped cache in the benchmark's configuration; four
    (batch, head) rows are checked over all 32768 tokens."""
    m = axr()
    w = W.llama_decode()
    B, Hkv, T, d = w["keys"].shape
    b, bits = w["b"], w["sign_bits"]
    Hq = w["q"].shape[1]
    packed, norms = m.quantize_keys(w["keys"].to(DEV), bits, b)
    scale = 1.0 / math.sqrt(d)
    probs, lse = m.score_softmax(w["q"].to(DEV), packed, norms, bits, b, scale=scale)
    torch.cuda.synchronize()
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(w["q"]), s)
    G = Hq // Hkv
    for bi, h in [(0, 0), (3, 17), (5, 30), (7, 31)]:
        kvh = h // G
        gidx = A.unpack_indices(words_u32(packed[bi, kvh]), d, b)[None, None]
        onorm = A.key_norms(f64(w["keys"][bi, kvh]))[None, None]
        qp = qprime[bi:bi + 1, h:h + 1]
        ref = A.lut_scores(qp, gidx, onorm, c)[0]
        cond = A.score_condition(qp, gidx, onorm, c)[0]
        assert_softmax(f64(probs[bi, h:h + 1]), f64(lse[bi, h:h + 1]), ref, cond, scale, T,
                       f"llama row ({bi}, {h})")


@pytest.mark.parametrize("i", range(12))
def test_softmax_random_shapes(i):
    """Seeded random shapes: d, b, key dtype, KV heads, group sizes with padded
    head slots, t_cap >= T, lengths anywhere in [-2, T + 40], scales."""
    rng = np.random.default_rng(8000 + i)
    d = int(rng.choice([128, 256, 512]))
    b = int(rng.integers(2, 5))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    Hkv = int(rng.integers(1, 4))
    T = int(rng.integers(1, 2500 if d < 512 else 1200))
    t_cap = T + int(rng.integers(0, 60))
    B = int(rng.integers(1, 5))
    lens = [int(v) for v in rng.integers(-2, T + 40, size=B)]
    dtype = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))]
    scale = float(rng.choice([1.0 / math.sqrt(d), 0.3, 1.0]))
    print(f"softmax random {i}: d={d} b={b} G={G} Hkv={Hkv} T={T} t_cap={t_cap} lens={lens} "
          f"{dtype} scale={scale}", flush=True)
    _run(d, b, G, lens, T=T, t_cap=t_cap, scale=scale, seed=9000 + i, Hkv=Hkv, dtype=dtype)
