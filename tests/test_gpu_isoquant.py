"""GPU parity of the comparison write path with block-quaternion rotations
("IsoQuant: Hardware-Aligned SO(4) Isoclinic Rotations for LLM KV Cache
Compression", Abstract: IsoQuant-Full q_L v conj(q_R), IsoQuant-Fast q_L v on
4-coordinate blocks) followed by the same Lloyd-Max quantizer: indices by the
boundary rule, norms, the exported transform within 1e-5, and the
reconstruction error of the three transforms on the write-sweep keys."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import axelram as A
from tests._parity import f64, words_u32, assert_indices, assert_norms, TRANSFORM_ATOL

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


def _check(keys_cpu, b, full, label, rows=None):
    m = axr()
    d = keys_cpu.shape[-1]
    qs = W.isoquant_quaternions(d)
    qdev = torch.from_numpy(qs).to(DEV)
    keys = keys_cpu.to(DEV)
    packed, norms = m.quantize_keys_isoquant(keys, qdev, b, full=full)
    y_gpu = m.transform_isoquant(keys, qdev, full=full, normalize=True)
    torch.cuda.synchronize()
    flat = keys_cpu.reshape(-1, d)
    rows = np.arange(flat.shape[0]) if rows is None else rows
    k64 = f64(flat[torch.from_numpy(rows)])
    q64 = qs.astype(np.float64)
    ql, qr = q64[:, 0], (q64[:, 1] if full else None)
    w = A.isoquant_write_path(k64, ql, qr, b)
    _, t = A.lloyd_max_codebook(d, b)
    gidx = A.unpack_indices(words_u32(packed.reshape(-1, packed.shape[-1]))[rows], d, b)
    assert_indices(gidx, w["idx"], w["y"], t, label)
    assert_norms(f64(norms.reshape(-1))[rows], w["norms"], label)
    assert np.max(np.abs(f64(y_gpu.reshape(-1, d))[rows] - w["y"])) <= TRANSFORM_ATOL, label
    return gidx, k64


@pytest.mark.parametrize("full", [True, False])
@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("d", [128, 256, 512])
def test_isoquant_write_ragged(d, b, dtype, full):
    rng = np.random.default_rng(3000 + d + 10 * b)
    n = 3 * 64 + 37
    k = rng.standard_normal((1, 1, n, d)) * np.exp(rng.standard_normal(d))
    k[0, 0, 5] = 0.0                                          # a zero key
    keys = torch.from_numpy(k.astype(np.float32)).to(dtype)
    _check(keys, b, full, f"isoquant d={d} b={b} {dtype} full={full}")


@pytest.mark.parametrize("full", [True, False])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_isoquant_tiny_and_huge_keys(dtype, full):
    """Keys whose squares underflow or overflow fp32 take their norm from the
    rotated coordinates, as in the Hadamard path."""
    rng = np.random.default_rng(3300)
    d, b, n = 128, 3, 256
    k = rng.standard_normal((1, 1, n, d))
    k[0, 0, 0::3] *= 1e-30
    k[0, 0, 1::3] *= 1e28
    keys = torch.from_numpy(k.astype(np.float32)).to(dtype)
    _check(keys, b, full, f"isoquant tiny/huge {dtype} full={full}")


@pytest.mark.parametrize("full", [True, False])
def test_isoquant_write_sweep_full_size_sampled(full):
    w = W.write_sweep(d=256, b=3)
    flat_n = w["keys"].numel() // 256
    _check(w["keys"], 3, full, f"write sweep d=256 full={full}",
           rows=W.sample_rows(flat_n, 2000))


def test_reconstruction_error_of_the_three_transforms():
    """Stage-1 quantize-dequantize error of unit vectors from the GPU's
    indices: each transform lands near Max's distortion for b = 3 on
    Gaussian keys (0.0345 per vector), the Hadamard path included."""
    m = axr()
    d, b = 128, 3
    w = W.write_sweep(d=d, b=b, T=2048)
    rows = np.arange(4096)
    c, _ = A.lloyd_max_codebook(d, b)
    out = {}
    for full in (True, False):
        gidx, k64 = _check(w["keys"], b, full, f"mse full={full}", rows=rows)
        q64 = W.isoquant_quaternions(d).astype(np.float64)
        ql, qr = q64[:, 0], (q64[:, 1] if full else None)
        out[full] = A.reconstruction_mse(k64, gidx, c, lambda y: A.isoquant_unrotate(y, ql, qr))
    packed, _ = m.quantize_keys(w["keys"].to(DEV), w["sign_bits"], b)
    torch.cuda.synchronize()
    gidx = A.unpack_indices(words_u32(packed.reshape(-1, packed.shape[-1])), d, b)[rows]
    s = A.signs_from_bits(w["sign_bits"])
    h = A.sylvester_hadamard(d)
    wht = A.reconstruction_mse(f64(w["keys"].reshape(-1, d))[rows], gidx, c,
                               lambda y: (y @ h) / np.sqrt(d) * s)
    for name, v in (("full", out[True]), ("fast", out[False]), ("wht", wht)):
        assert abs(v - 0.03455) < 0.003, f"{name}: {v}"
