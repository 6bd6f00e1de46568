"""GPU parity over seeded random shape combinations: (d, b, key and query
dtypes, batch, KV heads, GQA group size including ones that leave padded
head slots, context, allocated context t_cap > T, per-sequence lengths).
Every output of every case is checked against the oracle: indices within
the boundary window, norms, and scores (the ragged ones only up to each
row's length, with the rest of the output left untouched)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, assert_indices, assert_norms, assert_scores

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DTYPES = [torch.float32, torch.float16, torch.bfloat16]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lut_attention_scoring_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _config(i):
    rng = np.random.default_rng(4000 + i)
    d = int(rng.choice([128, 256, 512]))
    b = int(rng.integers(2, 5))
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24]))
    T = int(rng.integers(1, 2500 if d < 512 else 1200))
    t_cap = T + int(rng.integers(0, 40))
    kdt = DTYPES[int(rng.integers(0, 3))]
    qdt = DTYPES[int(rng.integers(0, 3))]
    ragged = bool(rng.integers(0, 2))
    return rng, d, b, B, Hkv, G, T, t_cap, kdt, qdt, ragged


@pytest.mark.parametrize("i", range(24))
def test_random_shape(i):
    import lut_attention_scoring_amd as axr
    rng, d, b, B, Hkv, G, T, t_cap, kdt, qdt, ragged = _config(i)
    label = f"case {i}: d={d} b={b} B={B} Hkv={Hkv} G={G} T={T} t_cap={t_cap} {kdt} {qdt} ragged={ragged}"
    print(label, flush=True)
    scale = np.exp(rng.standard_normal(d))      # outlier channels
    keys = torch.from_numpy((rng.standard_normal((B, Hkv, t_cap, d)) * scale).astype(np.float32)).to(kdt)
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32)).to(qdt)
    bits = W.sign_bits(d)
    packed, norms = axr.quantize_keys(keys.to(DEV), bits, b)
    lens = None
    if ragged:
        lens_np = rng.integers(-2, T + 5, size=B).astype(np.int32)
        lens = torch.from_numpy(lens_np).to(DEV)
    out = torch.full((B, Hkv * G, T), float("nan"), device=DEV)
    axr.score(q.to(DEV), packed, norms, bits, b, T=T, out=out, lens=lens)
    torch.cuda.synchronize()

    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(d, b)
    k64 = f64(keys.reshape(-1, d))
    y, onorm = A.transform_keys(k64, s)
    gidx = A.unpack_indices(words_u32(packed.reshape(-1, d * b // 32)), d, b)
    assert_indices(gidx, A.quantize(y, t), y, t, label)
    assert_norms(f64(norms.reshape(-1)), onorm, label)

    qprime = A.transform_queries(f64(q), s)
    gidx4 = gidx.reshape(B, Hkv, t_cap, d)[:, :, :T]
    onorm3 = onorm.reshape(B, Hkv, t_cap)[:, :, :T]
    got = f64(out)
    if lens is None:
        assert_scores(got, qprime, gidx4, onorm3, c, label)
    else:
        for bi in range(B):
            n = int(min(max(int(lens_np[bi]), 0), T))
            if n:
                assert_scores(got[bi:bi + 1, :, :n], qprime[bi:bi + 1], gidx4[bi:bi + 1, :, :n],
                              onorm3[bi:bi + 1, :, :n], c, f"{label} row {bi}")
            assert np.all(np.isnan(got[bi, :, n:])), f"{label}: row {bi} written past its length"
