"""GPU parity of the decode step ("AXELRAM: Quantize Once, Never Dequantize",
Abstract: a key is quantized once, when it is written, and read by table
lookup).  axr_append_keys writes one new key per (sequence, KV head) into its
cache slot; axr_score_ragged scores every sequence over its own length.  Both
are compared with the oracle: indices by the boundary rule, scores given the
GPU's own indices, and every slot or score that must not change is checked
bit for bit."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, assert_indices, assert_scores, assert_norms

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


def _keys(rng, shape, dtype, scale=2.0):
    return torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(dtype)


def _check_appended(new_cpu, packed_after, norms_after, pos, bits, b, label):
    """Records and norms at the appended slots against the oracle's write of
    the new keys [B, Hkv, d]."""
    d = new_cpu.shape[-1]
    t_cap = packed_after.shape[2]
    s = A.signs_from_bits(bits)
    _, t = A.lloyd_max_codebook(d, b)
    y, onorm = A.transform_keys(f64(new_cpu), s)
    oidx = A.quantize(y, t)
    pw = words_u32(packed_after)
    pn = f64(norms_after)
    n_checked = 0
    for bi, slot in enumerate(pos):
        if 0 <= slot < t_cap:
            gidx = A.unpack_indices(pw[bi, :, slot], d, b)
            assert_indices(gidx, oidx[bi], y[bi], t, f"{label} bi={bi}")
            assert_norms(pn[bi, :, slot], onorm[bi], f"{label} bi={bi}")
            n_checked += 1
    return n_checked


def _untouched(before_p, before_n, after_p, after_n, pos):
    """Every slot other than the appended ones is bit-identical."""
    t_cap = before_p.shape[2]
    keep = np.ones(before_p.shape[:3], dtype=bool)
    for bi, slot in enumerate(pos):
        if 0 <= slot < t_cap:
            keep[bi, :, slot] = False
    assert np.array_equal(before_p[keep], after_p[keep])
    assert np.array_equal(before_n[keep].view(np.uint32), after_n[keep].view(np.uint32))


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_append_into_slots(d, b, dtype):
    m = axr()
    rng = np.random.default_rng(1000 + 10 * d + b)
    B, Hkv, t_cap = 6, 3, 150
    bits = W.sign_bits(d)
    cache = _keys(rng, (B, Hkv, t_cap, d), dtype)
    packed, norms = m.quantize_keys(cache.to(DEV), bits, b)
    new = _keys(rng, (B, Hkv, d), dtype, scale=5.0)
    pos = [0, t_cap - 1, 57, -1, t_cap, 2]               # two slots outside [0, t_cap)
    torch.cuda.synchronize()
    before_p, before_n = words_u32(packed).copy(), norms.cpu().numpy().copy()
    m.append_keys(new.to(DEV), bits, b, packed, norms,
                  torch.tensor(pos, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    after_p, after_n = words_u32(packed), norms.cpu().numpy()
    assert _check_appended(new, packed, norms, pos, bits, b, f"append d={d} b={b}") == 4
    _untouched(before_p, before_n, after_p, after_n, pos)


@pytest.mark.parametrize("i", range(8))
def test_append_random_shapes(i):
    """Appends with seeded random batch and KV-head counts (up to several
    blocks of keys), cache lengths and slots anywhere in [-3, t_cap + 3)."""
    m = axr()
    rng = np.random.default_rng(7500 + i)
    d = int(rng.choice([128, 256, 512]))
    b = int(rng.integers(2, 5))
    dtype = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))]
    B = int(rng.integers(1, 41))
    Hkv = int(rng.integers(1, 9))
    t_cap = int(rng.integers(1, 64))
    pos = [int(v) for v in rng.integers(-3, t_cap + 3, size=B)]
    label = f"append random {i}: d={d} b={b} {dtype} B={B} Hkv={Hkv} t_cap={t_cap}"
    bits = W.sign_bits(d)
    cache = _keys(rng, (B, Hkv, t_cap, d), dtype)
    packed, norms = m.quantize_keys(cache.to(DEV), bits, b)
    new = _keys(rng, (B, Hkv, d), dtype, scale=5.0)
    torch.cuda.synchronize()
    before_p, before_n = words_u32(packed).copy(), norms.cpu().numpy().copy()
    m.append_keys(new.to(DEV), bits, b, packed, norms,
                  torch.tensor(pos, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    n_app = sum(1 for p_ in pos if 0 <= p_ < t_cap)
    assert _check_appended(new, packed, norms, pos, bits, b, label) == n_app
    _untouched(before_p, before_n, words_u32(packed), norms.cpu().numpy(), pos)


def test_append_zero_key_and_exact_ties():
    # a zero key takes the cell below 0 everywhere; its norm is 0
    m = axr()
    d, b, B, Hkv, t_cap = 128, 3, 2, 2, 8
    bits = W.sign_bits(d)
    packed = torch.zeros(B, Hkv, t_cap, d * b // 32, dtype=torch.int32, device=DEV)
    norms = torch.full((B, Hkv, t_cap), -1.0, device=DEV)
    new = torch.zeros(B, Hkv, d, dtype=torch.float16)
    new[1, 1, 3] = 1.0                                   # one basis key
    pos = [5, 0]
    m.append_keys(new.to(DEV), bits, b, packed, norms,
                  torch.tensor(pos, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    idx = A.unpack_indices(words_u32(packed[0, :, 5]), d, b)
    assert np.all(idx == (1 << (b - 1)) - 1)
    assert np.all(norms[0, :, 5].cpu().numpy() == 0.0)
    _check_appended(new, packed, norms, pos, bits, b, "zero/basis keys")


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("b", [2, 3, 4])
def test_score_ragged_lengths(G, b):
    m = axr()
    rng = np.random.default_rng(2000 + 10 * G + b)
    d, Hkv, t_cap, T = 128, 2, 1500, 1400
    lens = [0, 1, 777, T, 5000, -5, 255, 256]             # empty, single, tile edges, clamps
    B = len(lens)
    bits = W.sign_bits(d)
    keys = _keys(rng, (B, Hkv, t_cap, d), torch.float16)
    q = _keys(rng, (B, Hkv * G, d), torch.float16, scale=1.0)
    packed, norms = m.quantize_keys(keys.to(DEV), bits, b)
    out = torch.full((B, Hkv * G, T), SENTINEL, device=DEV)
    m.score(q.to(DEV), packed, norms, bits, b, T=T, out=out,
            lens=torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(q), s)
    got = f64(out)
    gidx_all = A.unpack_indices(words_u32(packed[:, :, :T]), d, b)
    onorm_all = A.key_norms(f64(keys[:, :, :T]))
    for bi, length in enumerate(lens):
        n_tok = min(max(length, 0), T)
        assert np.all(got[bi, :, n_tok:] == SENTINEL), f"bi={bi} wrote past its length"
        if n_tok:
            assert_scores(got[bi:bi + 1, :, :n_tok], qprime[bi:bi + 1],
                          gidx_all[bi:bi + 1, :, :n_tok], onorm_all[bi:bi + 1, :, :n_tok], c,
                          f"ragged G={G} b={b} bi={bi}")


def test_score_ragged_full_lengths_equal_dense_scores():
    m = axr()
    rng = np.random.default_rng(31)
    d, b, B, Hkv, G, T = 128, 3, 3, 2, 4, 3000
    bits = W.sign_bits(d)
    keys = _keys(rng, (B, Hkv, T, d), torch.float16)
    q = _keys(rng, (B, Hkv * G, d), torch.float16, scale=1.0).to(DEV)
    packed, norms = m.quantize_keys(keys.to(DEV), bits, b)
    dense = m.score(q, packed, norms, bits, b)
    ragged = m.score(q, packed, norms, bits, b,
                     lens=torch.full((B,), T, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(dense, ragged)


@pytest.mark.parametrize("b", [3, 4])
def test_decode_loop(b):
    """Four decode steps over sequences of different lengths: each step
    appends a key per (sequence, KV head) at the end of its sequence and
    scores the new query against everything written so far."""
    m = axr()
    rng = np.random.default_rng(40 + b)
    d, B, Hkv, G, t_cap = 128, 3, 2, 4, 700
    lens = np.array([100, 333, 690], dtype=np.int64)
    bits = W.sign_bits(d)
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    keys = _keys(rng, (B, Hkv, t_cap, d), torch.bfloat16)
    packed, norms = m.quantize_keys(keys.to(DEV), bits, b)
    for step in range(4):
        new = _keys(rng, (B, Hkv, d), torch.bfloat16)
        q = _keys(rng, (B, Hkv * G, d), torch.bfloat16, scale=1.0)
        pos = lens.copy()
        m.append_keys(new.to(DEV), bits, b, packed, norms,
                      torch.tensor(pos, dtype=torch.int32, device=DEV))
        for bi in range(B):
            keys[bi, :, pos[bi]] = new[bi]
        lens += 1
        out = torch.full((B, Hkv * G, t_cap), SENTINEL, device=DEV)
        m.score(q.to(DEV), packed, norms, bits, b, out=out,
                lens=torch.tensor(lens, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        _check_appended(new, packed, norms, pos.tolist(), bits, b, f"step {step}")
        got = f64(out)
        qprime = A.transform_queries(f64(q), s)
        for bi in range(B):
            n_tok = int(lens[bi])
            assert np.all(got[bi, :, n_tok:] == SENTINEL)
            gidx = A.unpack_indices(words_u32(packed[bi:bi + 1, :, :n_tok]), d, b)
            onorm = A.key_norms(f64(keys[bi:bi + 1, :, :n_tok]))
            assert_scores(got[bi:bi + 1, :, :n_tok], qprime[bi:bi + 1], gidx, onorm, c,
                          f"step {step} bi={bi}")


def test_decode_step_llama_full_size_sampled():
    """The LLaMA-3.1-8B-shaped cache (8 x 8 KV heads x 32768 tokens, 32 query
    heads, d=128, b=3) in the benchmark's decode-step configuration: append at
    ragged positions, then score each sequence up to its new length.  Checked
    on the appended slots and a token sample, which the oracle computes one by
    one."""
    m = axr()
    w = W.llama_decode()
    B, Hkv, T, d = w["keys"].shape
    b, bits = w["b"], w["sign_bits"]
    keys = w["keys"].to(DEV)
    packed, norms = m.quantize_keys(keys, bits, b)
    rng = np.random.default_rng(77)
    pos = rng.integers(T // 2, T, size=B)
    pos[0] = T - 1
    new = _keys(rng, (B, Hkv, d), torch.float16)
    m.append_keys(new.to(DEV), bits, b, packed, norms,
                  torch.tensor(pos, dtype=torch.int32, device=DEV))
    lens = torch.tensor(pos + 1, dtype=torch.int32, device=DEV)
    out = torch.full((B, w["q"].shape[1], T), SENTINEL, device=DEV)
    m.score(w["q"].to(DEV), packed, norms, bits, b, out=out, lens=lens)
    torch.cuda.synchronize()
    _check_appended(new, packed, norms, pos.tolist(), bits, b, "llama decode")
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(w["q"]), s)
    kc = w["keys"].clone()
    for bi in range(B):
        kc[bi, :, pos[bi]] = new[bi]
    toks = W.sample_rows(T, 96)
    for bi in range(B):
        n_tok = int(pos[bi]) + 1
        sel = np.unique(np.concatenate([toks[toks < n_tok], [n_tok - 1]]))
        tt = torch.from_numpy(sel)
        gidx = A.unpack_indices(words_u32(packed[bi:bi + 1, :, tt]), d, b)
        onorm = A.key_norms(f64(kc[bi:bi + 1, :, tt]))
        assert_scores(f64(out[bi:bi + 1, :, tt]), qprime[bi:bi + 1], gidx, onorm, c,
                      f"llama decode bi={bi}")
        after = f64(out[bi, :, n_tok:])
        assert np.all(after == SENTINEL)


# ---------------------------------------------------------------------------
# The fused decode step (axr_decode_step): append and score in one launch.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,b,G,dtype", [
    (128, 3, 4, torch.float16), (128, 2, 1, torch.float32), (128, 4, 8, torch.bfloat16),
    (128, 3, 16, torch.float16), (256, 3, 8, torch.float16), (512, 4, 4, torch.bfloat16),
    (512, 2, 8, torch.float32)])
def test_fused_decode_step(d, b, G, dtype):
    m = axr()
    rng = np.random.default_rng(5000 + d + 10 * b + G)
    Hkv, t_cap, T = 2, 2100, 2000
    # tile edges, -1, past T inside the cache, past t_cap
    pos = [0, 1999, 777, -1, 2050, 255, 256, 1023, t_cap + 3]
    B = len(pos)
    bits = W.sign_bits(d)
    cache = _keys(rng, (B, Hkv, t_cap, d), dtype)
    packed, norms = m.quantize_keys(cache.to(DEV), bits, b)
    new = _keys(rng, (B, Hkv, d), dtype, scale=4.0)
    q = _keys(rng, (B, Hkv * G, d), dtype, scale=1.0)
    out = torch.full((B, Hkv * G, T), SENTINEL, device=DEV)
    torch.cuda.synchronize()
    before_p, before_n = words_u32(packed).copy(), norms.cpu().numpy().copy()
    m.decode_step(q.to(DEV), new.to(DEV), bits, b, packed, norms,
                  torch.tensor(pos, dtype=torch.int32, device=DEV), T=T, out=out)
    torch.cuda.synchronize()
    label = f"fused d={d} b={b} G={G}"
    # appended records against the oracle's write of the new keys; all else untouched
    assert _check_appended(new, packed, norms, pos, bits, b, label) == 7
    _untouched(before_p, before_n, words_u32(packed), norms.cpu().numpy(), pos)
    # scores given the GPU's (new) records
    keys_now = cache.clone()
    for bi, slot in enumerate(pos):
        if 0 <= slot < t_cap:
            keys_now[bi, :, slot] = new[bi]
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(q), s)
    got = f64(out)
    for bi, slot in enumerate(pos):
        n_tok = min(max(slot + 1, 0), T)
        assert np.all(got[bi, :, n_tok:] == SENTINEL), f"{label} bi={bi} wrote past its length"
        if n_tok == 0:
            continue
        toks = np.unique(np.concatenate([np.arange(0, n_tok, 37), [n_tok - 1]]))
        tt = torch.from_numpy(toks)
        gidx = A.unpack_indices(words_u32(packed[bi:bi + 1, :, tt]), d, b)
        onorm = A.key_norms(f64(keys_now[bi:bi + 1, :, tt]))
        assert_scores(got[bi:bi + 1, :, toks], qprime[bi:bi + 1], gidx, onorm, c,
                      f"{label} bi={bi}")


def test_fused_decode_step_with_nothing_to_score():
    """T = 0: the fused step is the append alone (slots in and out of the
    cache), and the cache equals the one the write path's append gives."""
    m = axr()
    rng = np.random.default_rng(6100)
    d, b, Hkv, G, t_cap = 128, 3, 2, 4, 50
    pos = [0, 49, 50, -1, 17]
    B = len(pos)
    bits = W.sign_bits(d)
    cache = _keys(rng, (B, Hkv, t_cap, d), torch.float16)
    new = _keys(rng, (B, Hkv, d), torch.float16, scale=4.0)
    q = _keys(rng, (B, Hkv * G, d), torch.float16, scale=1.0)
    pos_t = torch.tensor(pos, dtype=torch.int32, device=DEV)
    packed, norms = m.quantize_keys(cache.to(DEV), bits, b)
    ref_p, ref_n = packed.clone(), norms.clone()
    m.append_keys(new.to(DEV), bits, b, ref_p, ref_n, pos_t)
    out = torch.empty(B, Hkv * G, 0, device=DEV)
    m.decode_step(q.to(DEV), new.to(DEV), bits, b, packed, norms, pos_t, T=0, out=out)
    torch.cuda.synchronize()
    assert torch.equal(packed, ref_p) and torch.equal(norms, ref_n)
    assert _check_appended(new, packed, norms, pos, bits, b, "fused T=0") == 3


@pytest.mark.parametrize("i", range(12))
def test_fused_decode_step_random(i):
    """The fused decode step on seeded random shapes: d, b, key dtype, KV
    heads, group size, t_cap >= T and slots anywhere in [-3, t_cap + 3)."""
    m = axr()
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([128, 256, 512]))
    b = int(rng.integers(2, 5))
    dtype = [torch.float32, torch.float16, torch.bfloat16][int(rng.integers(0, 3))]
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    t_cap = int(rng.integers(1, 1500))
    T = int(rng.integers(1, t_cap + 1))
    B = int(rng.integers(1, 6))
    pos = [int(v) for v in rng.integers(-3, t_cap + 3, size=B)]
    label = f"fused random {i}: d={d} b={b} {dtype} Hkv={Hkv} G={G} t_cap={t_cap} T={T} pos={pos}"
    print(label, flush=True)
    bits = W.sign_bits(d)
    cache = _keys(rng, (B, Hkv, t_cap, d), dtype)
    packed, norms = m.quantize_keys(cache.to(DEV), bits, b)
    new = _keys(rng, (B, Hkv, d), dtype, scale=4.0)
    q = _keys(rng, (B, Hkv * G, d), dtype, scale=1.0)
    out = torch.full((B, Hkv * G, T), SENTINEL, device=DEV)
    torch.cuda.synchronize()
    before_p, before_n = words_u32(packed).copy(), norms.cpu().numpy().copy()
    m.decode_step(q.to(DEV), new.to(DEV), bits, b, packed, norms,
                  torch.tensor(pos, dtype=torch.int32, device=DEV), T=T, out=out)
    torch.cuda.synchronize()
    n_app = sum(1 for p_ in pos if 0 <= p_ < t_cap)
    assert _check_appended(new, packed, norms, pos, bits, b, label) == n_app
    _untouched(before_p, before_n, words_u32(packed), norms.cpu().numpy(), pos)
    keys_now = cache.clone()
    for bi, slot in enumerate(pos):
        if 0 <= slot < t_cap:
            keys_now[bi, :, slot] = new[bi]
    s = A.signs_from_bits(bits)
    c, _ = A.lloyd_max_codebook(d, b)
    qprime = A.transform_queries(f64(q), s)
    got = f64(out)
    for bi, slot in enumerate(pos):
        n_tok = min(max(slot + 1, 0), T)
        assert np.all(got[bi, :, n_tok:] == SENTINEL), f"{label} bi={bi} wrote past its length"
        if n_tok == 0:
            continue
        tt = torch.arange(n_tok)
        gidx = A.unpack_indices(words_u32(packed[bi:bi + 1, :, tt]), d, b)
        onorm = A.key_norms(f64(keys_now[bi:bi + 1, :, tt]))
        assert_scores(got[bi:bi + 1, :, :n_tok], qprime[bi:bi + 1], gidx, onorm, c,
                      f"{label} bi={bi}")


@pytest.mark.parametrize("scale", [3e-30, 3e25])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_tiny_and_huge_new_keys(dtype, scale):
    """New keys whose squared entries underflow or overflow fp32, appended by
    the write kernel and by the fused decode step: records and norms as the
    oracle's."""
    m = axr()
    rng = np.random.default_rng(5151)
    d, b, Hkv, G, t_cap, T = 128, 3, 2, 4, 600, 600
    pos = [5, 599, 300]
    B = len(pos)
    bits = W.sign_bits(d)
    cache = _keys(rng, (B, Hkv, t_cap, d), dtype)
    new = _keys(rng, (B, Hkv, d), dtype, scale=scale)
    q = _keys(rng, (B, Hkv * G, d), dtype, scale=1.0)
    pos_t = torch.tensor(pos, dtype=torch.int32, device=DEV)
    for fused in (False, True):
        packed, norms = m.quantize_keys(cache.to(DEV), bits, b)
        if fused:
            m.decode_step(q.to(DEV), new.to(DEV), bits, b, packed, norms, pos_t, T=T)
        else:
            m.append_keys(new.to(DEV), bits, b, packed, norms, pos_t)
        torch.cuda.synchronize()
        assert _check_appended(new, packed, norms, pos, bits, b,
                               f"new keys at {scale:g} fused={fused}") == B


def test_fused_decode_step_matches_two_launches():
    """Fused and two-launch decode steps agree: records within the boundary
    rule (checked above), scores of every other token bit for bit, and the
    new token's score within the score bound."""
    m = axr()
    rng = np.random.default_rng(61)
    d, b, B, Hkv, G, t_cap = 128, 3, 4, 2, 4, 3000
    bits = W.sign_bits(d)
    cache = _keys(rng, (B, Hkv, t_cap, d), torch.float16).to(DEV)
    p1, n1 = m.quantize_keys(cache, bits, b)
    p2, n2 = p1.clone(), n1.clone()
    new = _keys(rng, (B, Hkv, d), torch.float16).to(DEV)
    q = _keys(rng, (B, Hkv * G, d), torch.float16, scale=1.0).to(DEV)
    pos = torch.tensor([2999, 100, 1500, 4095 % 3000], dtype=torch.int32, device=DEV)
    fused = m.decode_step(q, new, bits, b, p1, n1, pos)
    m.append_keys(new, bits, b, p2, n2, pos)
    two = m.score(q, p2, n2, bits, b, lens=pos + 1)
    torch.cuda.synchronize()
    for bi, slot in enumerate(pos.tolist()):
        assert torch.equal(fused[bi, :, :slot], two[bi, :, :slot])
    torch.testing.assert_close(n1, n2, rtol=1e-6, atol=0)
