"""The seeded generators are deterministic and have the stated shapes,
dtypes and value structure."""

import numpy as np
import torch

import workloads as W


def test_sign_bits_seeded():
    a, b = W.sign_bits(128), W.sign_bits(128)
    assert a.dtype == np.uint8 and a.shape == (128,)
    np.testing.assert_array_equal(a, b)
    assert set(np.unique(a)) <= {0, 1}
    assert not np.array_equal(W.sign_bits(128, seed=2), a)


def test_tiny():
    w = W.tiny()
    assert w["keys"].shape == (1, 1, 4096, 128) and w["keys"].dtype == torch.float32
    assert w["q"].shape == (1, 1, 128)
    assert torch.equal(w["keys"], W.tiny()["keys"])


def test_llama_decode_small_has_outlier_channels():
    w = W.llama_decode(B=2, Hkv=2, Hq=8, T=512)
    k = w["keys"].float()
    assert w["keys"].dtype == torch.float16 and k.shape == (2, 2, 512, 128)
    assert w["q"].shape == (2, 8, 128)
    rms = k.pow(2).mean(dim=(0, 2)).sqrt()           # per (head, channel)
    assert float(rms.max() / rms.min()) > 10.0       # log-normal channel scales
    assert torch.equal(w["keys"], W.llama_decode(B=2, Hkv=2, Hq=8, T=512)["keys"])


def test_qwen_layers_have_heterogeneous_norms():
    scales = [W.qwen_layer(l, B=1, Hkv=2, Hq=16, T=64)["layer_scale"] for l in range(36)]
    assert min(scales) >= 1.0 and max(scales) <= 100.0
    assert max(scales) / min(scales) > 10.0
    w = W.qwen_layer(3, B=2, Hkv=2, Hq=16, T=128)
    assert w["keys"].dtype == torch.float16 and w["keys"].shape == (2, 2, 128, 128)
    assert w["b"] == 4


def test_long_context_and_sweep_dtypes():
    w = W.long_context(T=256)
    assert w["keys"].dtype == torch.bfloat16 and w["q"].shape == (1, 64, 128)
    s = W.write_sweep(d=512, T=64)
    assert s["keys"].shape == (1, 8, 64, 512) and s["q"] is None


def test_sample_rows():
    r = W.sample_rows(1000, 10)
    assert r[0] == 0 and r[-1] == 999 and len(np.unique(r)) == len(r)
