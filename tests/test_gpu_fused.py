"""GPU parity of the one-launch write and read path, axr_quantize_score
("AXELRAM: Quantize Once, Never Dequantize", Abstract: a key is transformed
and quantized once, on write, and scored by table lookup on its stored
indices).  Its records, norms and scores must equal, bit for bit, those of
axr_quantize_keys followed by axr_score on the same inputs; on smaller shapes
they are also checked against the oracle (indices by the boundary rule,
norms, and scores given the GPU's own indices)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, assert_indices, assert_scores, assert_norms

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


def _inputs(rng, B, Hkv, Hq, T, dtype, scale=2.0):
    keys = torch.from_numpy((rng.standard_normal((B, Hkv, T, 128)) * scale).astype(np.float32))
    q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32))
    return keys.to(dtype), q.to(dtype)


def _same(keys, q, bits, b, label):
    """Fused launch against the two launches, bit for bit; returns the
    fused outputs (on the CPU)."""
    m = axr()
    kd, qd = keys.to(DEV), q.to(DEV)
    p2, n2 = m.quantize_keys(kd, bits, b)
    s2 = m.score(qd, p2, n2, bits, b)
    # outputs pre-filled with junk: every element must be written
    B, Hkv, T, _ = keys.shape
    pf = torch.full((B, Hkv, T, 128 * b // 32), -7, dtype=torch.int32, device=DEV)
    nf = torch.full((B, Hkv, T), float("nan"), device=DEV)
    sf = torch.full((B, q.shape[1], T), float("nan"), device=DEV)
    m.quantize_score(kd, qd, bits, b, packed=pf, norms=nf, out=sf)
    torch.cuda.synchronize()
    assert torch.equal(pf, p2), f"{label}: records differ"
    assert torch.equal(nf.view(torch.int32), n2.view(torch.int32)), f"{label}: norms differ"
    assert torch.equal(sf.view(torch.int32), s2.view(torch.int32)), f"{label}: scores differ"
    return pf.cpu(), nf.cpu(), sf.cpu()


SHAPES = [  # (B, Hkv, Hq, T)
    (2, 3, 12, 1000),    # G = 4, ragged tail
    (1, 2, 2, 17),       # G = 1, one full unit and one key
    (3, 1, 3, 5000),     # G = 3 (a padded head slot)
    (1, 4, 8, 16),       # G = 2, exactly one unit
    (1, 1, 1, 4096),     # the tiny workload's shape
    (2, 2, 8, 40000),    # several tiles per row
    (3, 2, 4, 1),        # one token per row
    (1, 3, 6, 5),        # fewer tokens than a unit
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("b", [2, 3])
@pytest.mark.parametrize("shape", SHAPES)
def test_fused_matches_two_launches(shape, b, dtype):
    B, Hkv, Hq, T = shape
    rng = np.random.default_rng(7000 + 97 * T + 13 * Hq + b)
    keys, q = _inputs(rng, B, Hkv, Hq, T, dtype)
    print(f"fused vs two launches {shape} b={b} {dtype}", flush=True)
    _same(keys, q, W.sign_bits(128), b, f"{shape} b={b} {dtype}")


SHAPES_G8 = [  # (B, Hkv, Hq, T): eight query heads per KV head, two tables per block
    (2, 2, 16, 1000),    # ragged tail
    (1, 1, 8, 17),       # one full unit and one key
    (1, 2, 16, 40000),   # several tiles per row
    (2, 1, 8, 1),        # one token per row
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("shape", SHAPES_G8)
def test_fused_g8_matches_two_launches(shape, dtype):
    B, Hkv, Hq, T = shape
    rng = np.random.default_rng(7400 + 97 * T + 13 * Hq)
    keys, q = _inputs(rng, B, Hkv, Hq, T, dtype)
    print(f"fused vs two launches, G = 8 {shape} {dtype}", flush=True)
    _same(keys, q, W.sign_bits(128), 3, f"G=8 {shape} {dtype}")


def test_fused_g8_against_oracle():
    B, Hkv, Hq, T = 1, 2, 16, 700
    rng = np.random.default_rng(7500)
    keys, q = _inputs(rng, B, Hkv, Hq, T, torch.bfloat16)
    bits = W.sign_bits(128)
    pf, nf, sf = _same(keys, q, bits, 3, "oracle G=8")
    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(128, 3)
    y, onorm = A.transform_keys(f64(keys), s)
    gidx = A.unpack_indices(words_u32(pf), 128, 3)
    assert_indices(gidx, A.quantize(y, t), y, t, "fused G=8")
    assert_norms(f64(nf), onorm, "fused G=8")
    assert_scores(f64(sf), A.transform_queries(f64(q), s), gidx, onorm, c, "fused G=8")


def test_fused_long_context_full_size():
    """The long-context cache at full size (1,048,576 bf16 keys, G = 8, b = 3):
    bit for bit the two launches, and sampled tokens against the oracle."""
    w = W.long_context(b=3)
    print("fused vs two launches, long-context cache", flush=True)
    bits, b, d = w["sign_bits"], w["b"], 128
    pf, nf, sf = _same(w["keys"], w["q"], bits, b, "long context full size")
    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(d, b)
    toks = torch.from_numpy(W.sample_rows(pf.shape[2], 1024))
    y, onorm = A.transform_keys(f64(w["keys"][:, :, toks]).reshape(-1, d), s)
    tidx = A.unpack_indices(words_u32(pf[:, :, toks]), d, b)
    assert_indices(tidx.reshape(-1, d), A.quantize(y, t), y, t, "long context, fused")
    tnorm = A.key_norms(f64(w["keys"][:, :, toks]))
    assert_scores(f64(sf[:, :, toks]), A.transform_queries(f64(w["q"]), s), tidx, tnorm, c,
                  "long context, fused")


@pytest.mark.parametrize("b", [2, 3])
def test_fused_against_oracle(b):
    B, Hkv, Hq, T = 2, 2, 8, 700
    rng = np.random.default_rng(7100 + b)
    keys, q = _inputs(rng, B, Hkv, Hq, T, torch.float16)
    bits = W.sign_bits(128)
    pf, nf, sf = _same(keys, q, bits, b, f"oracle b={b}")
    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(128, b)
    y, onorm = A.transform_keys(f64(keys), s)
    oidx = A.quantize(y, t)
    gidx = A.unpack_indices(words_u32(pf), 128, b)
    assert_indices(gidx, oidx, y, t, f"fused b={b}")
    assert_norms(f64(nf), onorm, f"fused b={b}")
    qp = A.transform_queries(f64(q), s)
    assert_scores(f64(sf), qp, gidx, onorm, c, f"fused b={b}")


@pytest.mark.parametrize("scale", [1e-25, 1e30])
def test_fused_extreme_magnitudes(scale):
    """Keys whose squares underflow or overflow fp32 (the norm is taken again
    from the scaled transformed coordinates), mixed with ordinary keys in the
    same waves."""
    rng = np.random.default_rng(7200)
    keys, q = _inputs(rng, 1, 2, 8, 300, torch.float32)
    keys[:, :, ::3] *= scale
    _same(keys, q, W.sign_bits(128), 3, f"extreme {scale}")


def test_fused_llama_full_size():
    """The LLaMA-shaped decode cache at full size (2,097,152 keys, the
    benchmark's step, in its launch configuration): bit for bit the two
    launches, and against the oracle on sampled keys (indices, norms) and
    sampled tokens (every query head's score, given the GPU's indices)."""
    w = W.llama_decode()
    print("fused vs two launches, LLaMA decode cache", flush=True)
    bits, b = w["sign_bits"], w["b"]
    pf, nf, sf = _same(w["keys"], w["q"], bits, b, "llama full size")
    d = 128
    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(d, b)
    flat = w["keys"].reshape(-1, d)
    rows = W.sample_rows(flat.shape[0], 8192)
    y, onorm = A.transform_keys(f64(flat[torch.from_numpy(rows)]), s)
    gidx = A.unpack_indices(words_u32(pf.reshape(-1, pf.shape[-1]))[rows], d, b)
    assert_indices(gidx, A.quantize(y, t), y, t, "llama full size, fused")
    assert_norms(f64(nf.reshape(-1))[rows], onorm, "llama full size, fused")
    toks = torch.from_numpy(W.sample_rows(pf.shape[2], 1024))
    tidx = A.unpack_indices(words_u32(pf[:, :, toks]), d, b)
    tnorm = A.key_norms(f64(w["keys"][:, :, toks]))
    assert_scores(f64(sf[:, :, toks]), A.transform_queries(f64(w["q"]), s), tidx, tnorm, c,
                  "llama full size, fused")


def test_fused_tiny_workload_oracle():
    """The tiny workload (fp32 keys, one head) in one launch against the oracle."""
    w = W.tiny()
    bits, b = w["sign_bits"], w["b"]
    pf, nf, sf = _same(w["keys"], w["q"], bits, b, "tiny")
    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(128, b)
    y, onorm = A.transform_keys(f64(w["keys"]), s)
    oidx = A.quantize(y, t)
    gidx = A.unpack_indices(words_u32(pf), 128, b)
    assert_indices(gidx, oidx, y, t, "tiny fused")
    assert_norms(f64(nf), onorm, "tiny fused")
    assert_scores(f64(sf), A.transform_queries(f64(w["q"]), s), gidx, onorm, c, "tiny fused")


@pytest.mark.parametrize("seed", range(12))
def test_fused_random_shapes(seed):
    """Seeded random shapes (batch, KV heads, group size up to 4, length, b,
    key and query dtypes) in one launch, bit for bit the two launches."""
    rng = np.random.default_rng(7300 + seed)
    B = int(rng.integers(1, 4))
    Hkv = int(rng.integers(1, 5))
    G = int(rng.integers(1, 5))
    T = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 3000)),
                        int(rng.integers(3000, 20000))]))
    b = int(rng.choice([2, 3]))
    kdt = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))]
    qdt = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))]
    scale = float(np.exp(rng.uniform(-3.0, 3.0)))
    keys = torch.from_numpy((rng.standard_normal((B, Hkv, T, 128)) * scale).astype(np.float32))
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, 128)).astype(np.float32))
    label = f"random seed={seed} B={B} Hkv={Hkv} G={G} T={T} b={b} {kdt} {qdt}"
    print(label, flush=True)
    _same(keys.to(kdt), q.to(qdt), W.sign_bits(128), b, label)
