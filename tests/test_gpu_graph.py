"""The decode step (append + ragged score) captured in a HIP graph through
torch.cuda.CUDAGraph: the library launches on the caller's stream, so the
capture records its kernels with their arguments.  The graph is replayed
several times with eager work in between (new keys written into the captured
input buffer) and every replay must equal the same calls made eagerly, bit for
bit (the kernels are deterministic)."""

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lut_attention_scoring_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def test_decode_step_graph_replays_match_eager():
    import lut_attention_scoring_amd as m
    rng = np.random.default_rng(55)
    d, b, B, Hkv, G, t_cap = 128, 3, 3, 2, 4, 1500
    bits = W.sign_bits(d)
    keys = torch.from_numpy(rng.standard_normal((B, Hkv, t_cap, d)).astype(np.float32)).to(
        torch.float16).to(DEV)
    q = torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32)).to(
        torch.float16).to(DEV)
    base_p, base_n = m.quantize_keys(keys, bits, b)
    pos = torch.tensor([700, 1499, 3], dtype=torch.int32, device=DEV)
    lens = pos + 1
    new = torch.empty(B, Hkv, d, dtype=torch.float16, device=DEV)
    packed, norms = base_p.clone(), base_n.clone()
    out = torch.zeros(B, Hkv * G, t_cap, device=DEV)

    def step(pk, nm, o):
        m.append_keys(new, bits, b, pk, nm, pos)
        m.score(q, pk, nm, bits, b, out=o, lens=lens)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(packed, norms, out)                       # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(packed, norms, out)
    for rep in range(3):
        fresh = rng.standard_normal((B, Hkv, d)).astype(np.float32) * (1 + rep)
        new.copy_(torch.from_numpy(fresh).to(torch.float16))   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ep, en = base_p.clone(), base_n.clone()
        eo = torch.zeros_like(out)
        step(ep, en, eo)
        torch.cuda.synchronize()
        assert torch.equal(packed, ep), f"replay {rep}: records"
        assert torch.equal(norms, en), f"replay {rep}: norms"
        n_ok = [int(x) for x in lens.tolist()]
        for bi in range(B):
            assert torch.equal(out[bi, :, :n_ok[bi]], eo[bi, :, :n_ok[bi]]), f"replay {rep}"


def test_quantize_score_graph_replays_match_eager():
    """The one-launch write and read path captured in a graph: each replay,
    after new keys and queries are written eagerly into the captured input
    buffers, equals the eager call bit for bit."""
    import lut_attention_scoring_amd as m
    rng = np.random.default_rng(56)
    d, b, B, Hkv, G, T = 128, 3, 2, 3, 4, 2500
    bits = W.sign_bits(d)
    keys = torch.empty(B, Hkv, T, d, dtype=torch.float16, device=DEV)
    q = torch.empty(B, Hkv * G, d, dtype=torch.float16, device=DEV)
    packed = torch.empty(B, Hkv, T, d * b // 32, dtype=torch.int32, device=DEV)
    norms = torch.empty(B, Hkv, T, dtype=torch.float32, device=DEV)
    out = torch.empty(B, Hkv * G, T, dtype=torch.float32, device=DEV)

    def fill(rep):
        keys.copy_(torch.from_numpy(
            (rng.standard_normal((B, Hkv, T, d)) * (1 + rep)).astype(np.float32)).to(torch.float16))
        q.copy_(torch.from_numpy(rng.standard_normal((B, Hkv * G, d)).astype(np.float32)).to(
            torch.float16))

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.quantize_score(keys, q, bits, b, packed=packed, norms=norms, out=out)   # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.quantize_score(keys, q, bits, b, packed=packed, norms=norms, out=out)
    for rep in range(3):
        fill(rep + 1)                                   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ep, en, eo = m.quantize_score(keys, q, bits, b)
        torch.cuda.synchronize()
        assert torch.equal(packed, ep), f"replay {rep}: records"
        assert torch.equal(norms.view(torch.int32), en.view(torch.int32)), f"replay {rep}: norms"
        assert torch.equal(out.view(torch.int32), eo.view(torch.int32)), f"replay {rep}: scores"
