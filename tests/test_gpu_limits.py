"""GPU parity at the largest row the boundary accepts: one (batch, KV head)
row of packed records just under 2 GiB, the limit of the 32-bit offsets the
score kernel addresses a row with (the write path itself indexes in 64
bits).  Keys are drawn on the device from a seeded generator; sampled tokens
(the first, the last and a random set, plus the row's final 64) are checked
against the oracle key by key: indices within the boundary window, norms,
and scores from the GPU's own indices."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, assert_indices, assert_norms, assert_scores

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lut_attention_scoring_amd  # noqa: F401  (fails loudly if the library is missing)
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d, b, G", [(128, 2, 4), (512, 4, 8)])
def test_largest_row(d, b, G):
    import lut_attention_scoring_amd as axr

    T = (2 ** 31 - 1) // (d * b // 8)            # records of the row < 2 GiB
    print(f"largest row: d={d} b={b} G={G} T={T}", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(2024 + d + b)
    keys = torch.randn(1, 1, T, d, device=DEV, dtype=torch.float16, generator=gen)
    rng = np.random.default_rng(d + b)
    q_cpu = torch.from_numpy(rng.standard_normal((1, G, d)).astype(np.float32))
    bits = W.sign_bits(d)
    packed, norms = axr.quantize_keys(keys, bits, b)
    scores = axr.score(q_cpu.to(DEV), packed, norms, bits, b)
    torch.cuda.synchronize()

    toks = np.unique(np.concatenate([W.sample_rows(T, 300, seed=d), np.arange(T - 64, T)]))
    tt = torch.from_numpy(toks).to(DEV)
    k_s = keys[0, 0].index_select(0, tt).cpu()
    w_s = packed[0, 0].index_select(0, tt).cpu()
    n_s = norms[0, 0].index_select(0, tt).cpu()
    s_s = scores[0].index_select(1, tt).cpu()
    del keys, packed, norms, scores
    torch.cuda.empty_cache()

    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(d, b)
    y, onorm = A.transform_keys(f64(k_s), s)
    gidx = A.unpack_indices(words_u32(w_s), d, b)
    assert_indices(gidx, A.quantize(y, t), y, t, f"largest row d={d} b={b}")
    assert_norms(f64(n_s), onorm, f"largest row d={d} b={b}")
    qprime = A.transform_queries(f64(q_cpu), s)
    assert_scores(f64(s_s)[None], qprime, gidx[None, None], onorm[None, None], c,
                  f"largest row d={d} b={b} scores")
