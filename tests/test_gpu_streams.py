"""The library keeps no device state between calls: write and score calls
issued concurrently from several host threads, each on its own stream
(default priority), give bit for bit what the same calls give one after
another on one stream."""

import threading

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


def _cases():
    out = []
    for i, (d, b, Hkv, G, T) in enumerate([(128, 3, 4, 4, 5000), (256, 4, 2, 8, 3001),
                                           (128, 2, 1, 16, 7777), (512, 3, 2, 2, 1234)]):
        rng = np.random.default_rng(600 + i)
        keys = torch.from_numpy(rng.standard_normal((2, Hkv, T, d)).astype(np.float32))
        q = torch.from_numpy(rng.standard_normal((2, Hkv * G, d)).astype(np.float32))
        out.append((keys.to(torch.bfloat16 if i % 2 else torch.float16).to(DEV),
                    q.to(DEV), W.sign_bits(d), b))
    return out


def test_concurrent_streams_and_threads_match_sequential():
    import lut_attention_scoring_amd as axr
    cases = _cases()
    ref = []
    for keys, q, bits, b in cases:
        packed, norms = axr.quantize_keys(keys, bits, b)
        ref.append((packed, norms, axr.score(q, packed, norms, bits, b)))
    torch.cuda.synchronize()

    results = [None] * len(cases)
    errors = []
    barrier = threading.Barrier(len(cases))

    def worker(i):
        try:
            keys, q, bits, b = cases[i]
            stream = torch.cuda.Stream(device=DEV)
            barrier.wait()
            with torch.cuda.stream(stream):
                outs = []
                for _ in range(4):
                    packed, norms = axr.quantize_keys(keys, bits, b)
                    outs.append((packed, norms, axr.score(q, packed, norms, bits, b)))
            stream.synchronize()
            results[i] = outs
        except Exception as exc:                 # reported by the main thread
            errors.append((i, repr(exc)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for i, outs in enumerate(results):
        for packed, norms, scores in outs:
            assert torch.equal(packed, ref[i][0]), f"case {i}: records differ"
            assert torch.equal(norms, ref[i][1]), f"case {i}: norms differ"
            assert torch.equal(scores, ref[i][2]), f"case {i}: scores differ"
