"""Seeded synthetic inputs shaped like the LLM workloads of the AXELRAM page.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no normalisation, transform, codebook or scoring).  Both
the HIP path and the CPU oracle receive exactly these arrays.

"AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638), Abstract,
evaluates on LLaMA-3.1-8B and Qwen2.5-3B and attributes sign-pattern
sensitivity to layer-wise norm heterogeneity.  No weights or datasets are used
here: the generators reproduce only tensor shapes and value statistics
(outlier channels, per-layer norm scales, heavy tails).

Every generator returns a dict with
    keys       torch tensor [B, Hkv, T, d] (CPU) in the workload's dtype
    q          torch tensor [B, Hq, d] (CPU) or None for write-only workloads
    sign_bits  numpy uint8 [d]; bit j set means the sign pattern has -1 at j
    b          bit width
"""

from __future__ import annotations

import numpy as np
import torch

SIGN_SEED = 1


def sign_bits(d: int, seed: int = SIGN_SEED) -> np.ndarray:
    """The sign pattern as d bits drawn from numpy's PCG64 with `seed`."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2, size=d).astype(np.uint8)


def _to(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)


def tiny(T: int = 4096, d: int = 128, b: int = 3, seed: int = 0):
    """One head, T keys and one query, fp32 i.i.d. N(0, 1) from one stream
    (keys first, then the query)."""
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((1, 1, T, d))
    q = rng.standard_normal((1, 1, d))
    return {"keys": torch.from_numpy(keys.astype(np.float32)),
            "q": torch.from_numpy(q.astype(np.float32)),
            "sign_bits": sign_bits(d), "b": b}


def llama_decode(B: int = 8, Hkv: int = 8, Hq: int = 32, T: int = 32768,
                 d: int = 128, b: int = 3, seed: int = 101):
    """LLaMA-3.1-8B-shaped GQA decode cache: fp16 keys z * exp(g), z ~ N(0,1)
    per entry and g ~ N(0,1) per (KV head, channel), shared over batch and
    tokens (log-normal channel scales give outlier channels); queries N(0,1)."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((Hkv, d))
    scale = np.exp(g).astype(np.float32)
    z = rng.standard_normal((B, Hkv, T, d), dtype=np.float32)
    z *= scale[None, :, None, :]
    keys = _to(z, torch.float16)
    del z
    q = _to(rng.standard_normal((B, Hq, d), dtype=np.float32), torch.float16)
    return {"keys": keys, "q": q, "sign_bits": sign_bits(d), "b": b}


QWEN_LAYERS = 36


def qwen_layer(layer: int, B: int = 16, Hkv: int = 2, Hq: int = 16, T: int = 16384,
               d: int = 128, b: int = 4, seed: int = 102, n_layers: int = QWEN_LAYERS):
    """One layer of a Qwen2.5-3B-shaped cache: keys z * S_l * j_t with z ~ N(0,1),
    a per-layer scale S_l = exp(U[ln 1, ln 100]) (layer-wise norm
    heterogeneity) and a per-token, per-head jitter j ~ U[0.8, 1.2]; fp16.
    Layer l draws from child l of SeedSequence(seed)."""
    if not 0 <= layer < n_layers:
        raise ValueError("layer out of range")
    child = np.random.SeedSequence(seed).spawn(n_layers)[layer]
    rng = np.random.default_rng(child)
    s_l = float(np.exp(rng.uniform(0.0, np.log(100.0))))
    jitter = rng.uniform(0.8, 1.2, size=(B, Hkv, T, 1)).astype(np.float32)
    z = rng.standard_normal((B, Hkv, T, d), dtype=np.float32)
    z *= jitter * np.float32(s_l)
    keys = _to(z, torch.float16)
    del z
    q = _to(rng.standard_normal((B, Hq, d), dtype=np.float32), torch.float16)
    return {"keys": keys, "q": q, "sign_bits": sign_bits(d), "b": b, "layer_scale": s_l}


def long_context(B: int = 1, Hkv: int = 8, Hq: int = 64, T: int = 131072,
                 d: int = 128, b: int = 3, seed: int = 103):
    """Long-context cache: bf16 keys with i.i.d. Student-t (nu = 3) entries in
    every channel (heavy tails); queries N(0,1) in bf16."""
    rng = np.random.default_rng(seed)
    keys = _to(rng.standard_t(3.0, size=(B, Hkv, T, d)).astype(np.float32), torch.bfloat16)
    q = _to(rng.standard_normal((B, Hq, d), dtype=np.float32), torch.bfloat16)
    return {"keys": keys, "q": q, "sign_bits": sign_bits(d), "b": b}


def write_sweep(d: int = 128, b: int = 3, B: int = 1, Hkv: int = 8, T: int = 32768,
                seed: int = 104):
    """Prefill write: bf16 i.i.d. N(0,1) keys for T tokens x Hkv heads."""
    rng = np.random.default_rng(seed)
    keys = _to(rng.standard_normal((B, Hkv, T, d), dtype=np.float32), torch.bfloat16)
    return {"keys": keys, "q": None, "sign_bits": sign_bits(d), "b": b}


SIGN_CANDIDATES = 200
CALIBRATION_SAMPLES = 8


def sign_candidates(d: int, count: int = SIGN_CANDIDATES, seed: int = 105) -> np.ndarray:
    """Candidate sign patterns for the one-time selection, as bits [count, d]:
    candidate 0 is the default pattern (seed 1), candidate i > 0 draws d bits
    from PCG64 seeded with (seed, i)."""
    out = np.empty((count, d), dtype=np.uint8)
    out[0] = sign_bits(d)
    for i in range(1, count):
        out[i] = np.random.default_rng([seed, i]).integers(0, 2, size=d)
    return out


def calibration_samples(count: int = CALIBRATION_SAMPLES, B: int = 1, Hkv: int = 2,
                        Hq: int = 16, T: int = 2048, d: int = 128, seed: int = 106):
    """Calibration set for the sign-pattern selection: `count` synthetic layers
    shaped like the Qwen2.5-3B layers (per-layer norm scale exp(U[ln 1,
    ln 100]), per-token jitter U[0.8, 1.2]) with log-normal channel scales
    exp(g), g ~ N(0,1) per (KV head, channel), and a mean vector mu ~ N(0,1)
    per (KV head, channel) shared over tokens (keys of real layers are not
    centred; without a shared direction every sign pattern is equivalent):
        keys = (z * exp(g) + mu) * S_l * j,  z ~ N(0, 1);  q ~ N(0, 1).
    Returns keys [count, B, Hkv, T, d] and q [count, B, Hq, d], fp16."""
    children = np.random.SeedSequence(seed).spawn(count)
    keys = np.empty((count, B, Hkv, T, d), dtype=np.float32)
    q = np.empty((count, B, Hq, d), dtype=np.float32)
    scales = []
    for i, child in enumerate(children):
        rng = np.random.default_rng(child)
        s_l = float(np.exp(rng.uniform(0.0, np.log(100.0))))
        g = rng.standard_normal((Hkv, d))
        mu = rng.standard_normal((Hkv, d))
        jitter = rng.uniform(0.8, 1.2, size=(B, Hkv, T, 1))
        z = rng.standard_normal((B, Hkv, T, d))
        keys[i] = (z * np.exp(g)[None, :, None, :] + mu[None, :, None, :]) * jitter * s_l
        q[i] = rng.standard_normal((B, Hq, d))
        scales.append(s_l)
    return {"keys": _to(keys, torch.float16), "q": _to(q, torch.float16),
            "layer_scale": np.array(scales)}


def isoquant_quaternions(d: int, seed: int = 107) -> np.ndarray:
    """Per-block quaternion pairs for the block-rotation comparison transform:
    [d/4, 2, 4] float32, (q_left, q_right) of block m, each a Gaussian 4-vector
    divided by its length (a uniformly random unit quaternion)."""
    g = np.random.default_rng(seed).standard_normal((d // 4, 2, 4))
    return (g / np.linalg.norm(g, axis=-1, keepdims=True)).astype(np.float32)


# The five workloads at full size, by name.
FULL_SIZES = {
    "tiny_d128_b3_n4096": dict(B=1, Hkv=1, Hq=1, T=4096, d=128, b=3, dtype="f32"),
    "llama31_8b_gqa_decode_d128_b3": dict(B=8, Hkv=8, Hq=32, T=32768, d=128, b=3, dtype="f16"),
    "qwen25_3b_layer_sweep_d128_b4": dict(L=36, B=16, Hkv=2, Hq=16, T=16384, d=128, b=4,
                                          dtype="f16"),
    "long_context_t131072_d128": dict(B=1, Hkv=8, Hq=64, T=131072, d=128, bits=(2, 3, 4),
                                      dtype="bf16"),
    "write_sweep_t32768x8": dict(B=1, Hkv=8, T=32768, ds=(128, 256, 512), bits=(2, 3, 4),
                                 dtype="bf16"),
}


def sample_rows(n: int, count: int, seed: int = 7) -> np.ndarray:
    """Sorted distinct row indices for sampled checks: the first and last rows
    plus `count` rows drawn without replacement."""
    rng = np.random.default_rng(seed)
    count = min(count, n)
    pick = rng.choice(n, size=count, replace=False)
    pick = np.unique(np.concatenate([pick, [0, n - 1]]))
    return pick.astype(np.int64)
