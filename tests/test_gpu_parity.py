"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases run the oracle on every output; they span several tiles and a
ragged tail.  Full-size workloads run in the same launch configuration as the
benchmark and are checked on sampled keys and tokens, which the oracle
computes one by one."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import (f64, words_u32, assert_indices, assert_scores, assert_norms,
                           TRANSFORM_ATOL)

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


def _write_and_check(keys_cpu, bits, b, label, sample=None):
    """Quantize keys_cpu [B, Hkv, T, d] on the GPU and compare with the oracle
    on all keys (sample=None) or on a row sample.  Returns GPU (packed, norms)."""
    m = axr()
    d = keys_cpu.shape[-1]
    keys = keys_cpu.to(DEV)
    packed, norms = m.quantize_keys(keys, bits, b)
    y_gpu = m.transform(keys, bits, normalize=True)
    torch.cuda.synchronize()
    flat = keys_cpu.reshape(-1, d)
    rows = np.arange(flat.shape[0]) if sample is None else W.sample_rows(flat.shape[0], sample)
    k64 = f64(flat[torch.from_numpy(rows)])
    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(d, b)
    y, onorm = A.transform_keys(k64, s)
    oidx = A.quantize(y, t)
    gw = words_u32(packed.reshape(-1, packed.shape[-1]))[rows]
    gidx = A.unpack_indices(gw, d, b)
    assert_indices(gidx, oidx, y, t, label)
    assert_norms(f64(norms.reshape(-1))[rows], onorm, label)
    ygpu = f64(y_gpu.reshape(-1, d))[rows]
    assert np.max(np.abs(ygpu - y)) <= TRANSFORM_ATOL, label
    return packed, norms


def _score_and_check(q_cpu, keys_cpu, packed, norms, bits, b, label, T=None, sample=None):
    m = axr()
    d = q_cpu.shape[-1]
    q = q_cpu.to(DEV)
    Bn, Hq, _ = q_cpu.shape
    Hkv = packed.shape[1]
    T = packed.shape[2] if T is None else T
    scores = m.score(q, packed, norms, bits, b, T=T)
    qt = m.transform(q, bits, normalize=False)
    torch.cuda.synchronize()
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(q_cpu), s)
    qn = np.linalg.norm(f64(q_cpu), axis=-1)
    assert np.all(np.abs(f64(qt) - qprime) <= TRANSFORM_ATOL * qn[..., None]), label
    toks = np.arange(T) if sample is None else W.sample_rows(T, sample)
    tt = torch.from_numpy(toks)
    gidx = A.unpack_indices(words_u32(packed[:, :, tt]), d, b)
    onorm = A.key_norms(f64(keys_cpu[:, :, tt]))
    gs = f64(scores[:, :, tt])
    return assert_scores(gs, qprime, gidx, onorm, c, label)


# ---------------------------------------------------------------------------
# Tiny workload in full: d=128, b=3, one head, 4096 fp32 keys, one query.
# ---------------------------------------------------------------------------

def test_tiny_full():
    w = W.tiny()
    packed, norms = _write_and_check(w["keys"], w["sign_bits"], 3, "tiny")
    _score_and_check(w["q"], w["keys"], packed, norms, w["sign_bits"], 3, "tiny")


# ---------------------------------------------------------------------------
# Small, ragged, multi-tile cases over every (d, b, dtype).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_write_ragged(d, b, dtype):
    rng = np.random.default_rng(d * 10 + b)
    n = 3 * 64 + 37                                         # not a multiple of any block
    k = rng.standard_normal((1, 1, n, d)) * np.exp(rng.standard_normal(d))
    keys = torch.from_numpy(k.astype(np.float32)).to(dtype)
    _write_and_check(keys, W.sign_bits(d), b, f"write d={d} b={b} {dtype}")


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("b", [2, 3, 4])
def test_score_ragged_gqa(G, b):
    d, Bn, Hkv, T, t_cap = 128, 2, 2, 1237, 1300
    rng = np.random.default_rng(100 * G + b)
    keys = torch.from_numpy((rng.standard_normal((Bn, Hkv, t_cap, d)) * 3.0).astype(np.float32)
                            ).to(torch.float16)
    q = torch.from_numpy(rng.standard_normal((Bn, Hkv * G, d)).astype(np.float32)).to(torch.float16)
    bits = W.sign_bits(d)
    packed, norms = _write_and_check(keys, bits, b, f"gqa G={G}")
    _score_and_check(q, keys, packed, norms, bits, b, f"score G={G} b={b}", T=T)


@pytest.mark.parametrize("d,b", [(256, 2), (256, 3), (256, 4), (512, 2), (512, 3), (512, 4)])
def test_score_wide_heads(d, b):
    Bn, Hkv, G, T = 1, 2, 4, 777
    rng = np.random.default_rng(d + b)
    keys = torch.from_numpy(rng.standard_normal((Bn, Hkv, T, d)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((Bn, Hkv * G, d)).astype(np.float32)).to(torch.bfloat16)
    bits = W.sign_bits(d)
    packed, norms = _write_and_check(keys, bits, b, f"wide d={d}")
    _score_and_check(q, keys, packed, norms, bits, b, f"wide score d={d} b={b}")


@pytest.mark.parametrize("G,b", [(4, 3), (8, 2), (8, 4)])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 1023, 1024, 1025, 4097])
def test_score_unit_and_tile_edges(T, G, b):
    """Blocks hand out 16-token units from a counter: lengths one short of,
    equal to and one past a unit and a 1024-token tile, a tile holding a
    single token, and caches longer than the scored prefix."""
    d, Bn, Hkv = 128, 1, 1
    rng = np.random.default_rng(7000 + T + 10 * G + b)
    t_cap = T + 5
    keys = torch.from_numpy(rng.standard_normal((Bn, Hkv, t_cap, d)).astype(np.float32)
                            ).to(torch.float16)
    q = torch.from_numpy(rng.standard_normal((Bn, Hkv * G, d)).astype(np.float32)).to(torch.float16)
    bits = W.sign_bits(d)
    packed, norms = _write_and_check(keys, bits, b, f"edges T={T}")
    _score_and_check(q, keys, packed, norms, bits, b, f"edges score T={T} G={G} b={b}", T=T)


# ---------------------------------------------------------------------------
# Edge cases.
# ---------------------------------------------------------------------------

def test_empty_and_single():
    m = axr()
    bits = W.sign_bits(128)
    keys = torch.empty(0, 128, dtype=torch.float16, device=DEV)
    packed, norms = m.quantize_keys(keys, bits, 3)
    assert packed.shape == (0, 12) and norms.shape == (0,)
    q = torch.ones(1, 4, 128, dtype=torch.float16, device=DEV)
    out = m.score(q, torch.empty(1, 1, 0, 12, dtype=torch.int32, device=DEV),
                  torch.empty(1, 1, 0, device=DEV), bits, 3)
    assert out.shape == (1, 4, 0)
    one = torch.randn(1, 1, 1, 128, generator=torch.Generator().manual_seed(3)).to(torch.float16)
    p1, n1 = _write_and_check(one, bits, 3, "single key")
    _score_and_check(q.cpu(), one, p1, n1, bits, 3, "single key score")


def test_zero_norm_keys():
    m = axr()
    bits = W.sign_bits(128)
    keys = torch.zeros(1, 1, 70, 128, dtype=torch.float32)
    keys[0, 0, 3, 5] = 1.0                    # one basis vector among zero keys
    for b in (2, 3, 4):
        packed, norms = _write_and_check(keys, bits, b, f"zero keys b={b}")
        idx = A.unpack_indices(words_u32(packed[0, 0]), 128, b)
        zero_rows = [i for i in range(70) if i != 3]
        assert np.all(idx[zero_rows] == 2 ** (b - 1) - 1)
        assert float(norms[0, 0, 0]) == 0.0
        q = torch.randn(1, 2, 128, generator=torch.Generator().manual_seed(b))
        sc = m.score(q.to(DEV), packed, norms, bits, b)
        torch.cuda.synchronize()
        assert torch.all(sc[0, :, zero_rows] == 0.0)


def test_exact_cancellation_keys():
    """A constant key transforms to a vector with many exact zeros (ties at the
    middle threshold).  The GPU keeps them exactly 0 and takes the lower cell;
    the dense fp64 oracle leaves ~1e-17 of rounding and may go either way.
    Every disagreement must lie inside the boundary window; the 1e-4 count
    cap is for non-degenerate data and is not applied here."""
    m = axr()
    bits = W.sign_bits(128)
    keys = torch.ones(1, 1, 8, 128, dtype=torch.float32) * torch.arange(1, 9).view(1, 1, 8, 1)
    packed, norms = m.quantize_keys(keys.to(DEV), bits, 3)
    torch.cuda.synchronize()
    s = A.signs_from_bits(bits)
    c, t = A.lloyd_max_codebook(128, 3)
    y, _ = A.transform_keys(f64(keys.reshape(-1, 128)), s)
    oidx = A.quantize(y, t)
    gidx = A.unpack_indices(words_u32(packed.reshape(-1, 12)), 128, 3)
    bad = gidx != oidx
    assert np.all(np.abs(y[bad]) < 1e-12)
    assert np.all(gidx[np.abs(y) < 1e-12] == 3)


def test_extreme_magnitudes_fp32():
    rng = np.random.default_rng(77)
    k = rng.standard_normal((1, 1, 300, 128))
    k[0, 0, :100] *= 1e18
    k[0, 0, 100:200] *= 1e-18
    keys = torch.from_numpy(k.astype(np.float32))
    bits = W.sign_bits(128)
    packed, norms = _write_and_check(keys, bits, 3, "extreme magnitudes")
    q = torch.from_numpy(rng.standard_normal((1, 3, 128)).astype(np.float32))
    _score_and_check(q, keys, packed, norms, bits, 3, "extreme magnitudes score")


@pytest.mark.parametrize("G", [4, 8])
def test_query_magnitude_edges(G):
    """The table's fixed-point scale is chosen per head from the query: a
    zero query scores exactly 0, and tiny (1e-36), single-coordinate and huge
    (1e30) fp32 queries keep the score bound (scales beyond 2^126 are applied
    as two exact factors)."""
    d, b, T = 128, 3, 1500
    rng = np.random.default_rng(4242 + G)
    keys = torch.from_numpy(rng.standard_normal((1, 1, T, d)).astype(np.float32)).to(torch.float16)
    q = rng.standard_normal((1, G, d))
    q[0, 0] = 0.0
    q[0, 1] *= 1e-36
    q[0, 2] = 0.0
    q[0, 2, 7] = 1e-30
    q[0, 3] *= 1e30
    if G == 8:
        q[0, 4] *= 1e-20
        q[0, 5] *= 1e20
        q[0, 6] = 0.0
        q[0, 6, 100] = -3.0
    qt = torch.from_numpy(q.astype(np.float32))
    bits = W.sign_bits(d)
    packed, norms = _write_and_check(keys, bits, b, f"q edges G={G}")
    _score_and_check(qt, keys, packed, norms, bits, b, f"q edges score G={G}")
    scores = axr().score(qt.to(DEV), packed, norms, bits, b)
    torch.cuda.synchronize()
    assert torch.all(scores[0, 0] == 0), "a zero query must score exactly 0"


@pytest.mark.parametrize("b", [3, 4])
@pytest.mark.parametrize("d", [128, 512])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("scale", [1e-25, 1e-33, 1e25, 1e30])
def test_tiny_and_huge_keys(scale, dtype, d, b):
    """Keys whose squared entries underflow or overflow fp32, mixed token by
    token with ordinary keys (both paths in one wave): the norm comes from
    the transformed coordinates, so indices, norms and scores meet the same
    bounds as for any key.  At b = 4, norms outside [2^-100, 2^100] (the
    1e-33 and 1e30 keys) take the threshold search instead of the cell
    table, for their whole wave."""
    Hkv, G, T = 2, 4, 700
    rng = np.random.default_rng(int(abs(np.log10(scale))) + d + (scale > 1) + 1000 * (b - 3))
    k = rng.standard_normal((1, Hkv, T, d))
    k[:, :, ::2] *= scale
    keys = torch.from_numpy(k.astype(np.float32)).to(dtype)
    q = torch.from_numpy(rng.standard_normal((1, Hkv * G, d)).astype(np.float32))
    bits = W.sign_bits(d)
    label = f"keys at {scale:g} {dtype} d={d}"
    packed, norms = _write_and_check(keys, bits, b, label)
    _score_and_check(q, keys, packed, norms, bits, b, label)


@pytest.mark.parametrize("b", [3, 4])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_threshold_and_cell_sweep(d, b):
    """3-bit (threshold search) and 4-bit (cell table) quantizers: unit keys
    built so that their transformed coordinates are chosen values
    (k = s * (H v) gives y = v for a unit v):
    a dense sweep over +-3.2 sigma (every cell of the table in that range, a
    few hundred points per cell), points at and within 1e-7..1e-3 of every
    threshold on both sides, and basis keys (y = +-1, the table's ends).
    Indices off by one are allowed only inside the boundary window."""
    per_key = 8
    sigma = 1.0 / np.sqrt(d)
    c, t = A.lloyd_max_codebook(d, b)
    targets = list(np.linspace(-3.2 * sigma, 3.2 * sigma, 8192))
    for th in t:
        for off in (0.0, 1e-7, 3e-7, 1e-6, 2e-6, 1e-5, 1e-4, 1e-3):
            targets += [th + off, th - off]
    targets = np.array(targets)
    rng = np.random.default_rng(900 + d + 7 * b)
    rng.shuffle(targets)
    nkeys = (len(targets) + per_key - 1) // per_key
    v = np.zeros((nkeys + 2 * 4, d))
    for i in range(nkeys):
        pv = targets[i * per_key:(i + 1) * per_key]
        pos = rng.choice(d, size=len(pv), replace=False)
        rest = np.setdiff1d(np.arange(d), pos)
        v[i, pos] = pv
        v[i, rest] = np.sqrt((1.0 - np.sum(pv ** 2)) / len(rest)) * rng.choice([-1.0, 1.0], len(rest))
    for j, col in enumerate((0, 1, d // 2, d - 1)):
        v[nkeys + 2 * j, col] = 1.0
        v[nkeys + 2 * j + 1, col] = -1.0
    bits = W.sign_bits(d)
    s = A.signs_from_bits(bits)
    k = s * (v @ A.sylvester_hadamard(d))
    keys = torch.from_numpy(k.astype(np.float32)).reshape(1, 1, -1, d)
    m = axr()
    packed, norms = m.quantize_keys(keys.to(DEV), bits, b)
    torch.cuda.synchronize()
    y, onorm = A.transform_keys(f64(keys.reshape(-1, d)), s)
    assert np.max(np.abs(y - v)) < 1e-6
    oidx = A.quantize(y, t)
    gidx = A.unpack_indices(words_u32(packed.reshape(-1, d * b // 32)), d, b)
    bad = gidx != oidx
    if bad.any():
        dist = np.min(np.abs(y[bad][:, None] - t[None, :]), axis=1)
        assert dist.max() < 1e-6, f"d={d} b={b}: index off {dist.max():.3e} from any threshold"
        assert np.all(np.abs(gidx[bad] - oidx[bad]) == 1)
    far = np.min(np.abs(y[..., None] - t), axis=-1) >= 1e-6
    assert far.sum() > 0.9 * far.size
    assert np.array_equal(gidx[far], oidx[far])
    assert_norms(f64(norms.reshape(-1)), onorm, f"sweep d={d} b={b}")


@pytest.mark.parametrize("d, b, G", [(128, 3, 64), (128, 3, 63), (128, 4, 40), (128, 2, 33),
                                     (256, 3, 64), (512, 2, 33)])
def test_score_largest_groups(d, b, G):
    """Group sizes up to the supported 64 query heads per KV head, including
    ones that leave padded head slots in the last head group of a block."""
    rng = np.random.default_rng(6600 + d + b + G)
    Hkv, T = 2, 700
    keys = torch.from_numpy(rng.standard_normal((1, Hkv, T, d)).astype(np.float32)).to(
        torch.float16)
    q = torch.from_numpy(rng.standard_normal((1, Hkv * G, d)).astype(np.float32))
    bits = W.sign_bits(d)
    label = f"groups d={d} b={b} G={G}"
    packed, norms = _write_and_check(keys, bits, b, label)
    _score_and_check(q, keys, packed, norms, bits, b, label)


def test_score_is_deterministic_and_tile_independent():
    m = axr()
    w = W.llama_decode(B=1, Hkv=2, Hq=8, T=5000)
    keys = w["keys"].to(DEV)
    q = w["q"].to(DEV)
    packed, norms = m.quantize_keys(keys, w["sign_bits"], 3)
    a = m.score(q, packed, norms, w["sign_bits"], 3)
    b_ = m.score(q, packed, norms, w["sign_bits"], 3)
    # a prefix of the cache (different tiling) gives the same leading scores
    c = m.score(q, packed, norms, w["sign_bits"], 3, T=1234)
    torch.cuda.synchronize()
    assert torch.equal(a, b_)
    assert torch.equal(a[:, :, :1234], c)


# ---------------------------------------------------------------------------
# The five workloads.  Reduced sizes run the same recipe everywhere; full
# sizes run in the benchmark's launch configuration on sampled outputs.
# ---------------------------------------------------------------------------

def test_llama_decode_reduced_full_check():
    w = W.llama_decode(B=2, Hkv=8, Hq=32, T=600)
    packed, norms = _write_and_check(w["keys"], w["sign_bits"], 3, "llama reduced")
    _score_and_check(w["q"], w["keys"], packed, norms, w["sign_bits"], 3, "llama reduced")


def test_llama_decode_full_size_sampled():
    w = W.llama_decode()
    packed, norms = _write_and_check(w["keys"], w["sign_bits"], 3, "llama full", sample=8192)
    _score_and_check(w["q"], w["keys"], packed, norms, w["sign_bits"], 3, "llama full",
                     sample=1024)


def test_qwen_all_layers_reduced():
    for layer in range(W.QWEN_LAYERS):
        w = W.qwen_layer(layer, B=2, T=256)
        packed, norms = _write_and_check(w["keys"], w["sign_bits"], 4, f"qwen layer {layer}")
        _score_and_check(w["q"], w["keys"], packed, norms, w["sign_bits"], 4,
                         f"qwen layer {layer}")


@pytest.mark.parametrize("layer", [0, 35])
def test_qwen_layer_full_size_sampled(layer):
    w = W.qwen_layer(layer)
    packed, norms = _write_and_check(w["keys"], w["sign_bits"], 4, f"qwen full {layer}",
                                     sample=4096)
    _score_and_check(w["q"], w["keys"], packed, norms, w["sign_bits"], 4, f"qwen full {layer}",
                     sample=512)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_long_context_full_size_sampled(b):
    w = W.long_context(b=b)
    packed, norms = _write_and_check(w["keys"], w["sign_bits"], b, f"long b={b}", sample=4096)
    _score_and_check(w["q"], w["keys"], packed, norms, w["sign_bits"], b, f"long b={b}",
                     sample=256)


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_write_sweep_full_size_sampled(d, b):
    w = W.write_sweep(d=d, b=b)
    _write_and_check(w["keys"], w["sign_bits"], b, f"sweep d={d} b={b}", sample=4096)
