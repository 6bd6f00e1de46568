"""The Python binding checks what it hands to the C ABI as raw pointers:
dtypes and shapes of caller-supplied outputs (a wrong one would be written
through as another type, or past its end), then that every tensor is a
contiguous GPU tensor.  The dtype and shape checks come first, so they are
exercised here with CPU tensors."""

import pytest
import torch

import lut_attention_scoring_amd as axr
import workloads as W

BITS = W.sign_bits(128)


def test_quantize_output_dtypes():
    keys = torch.zeros(4, 128, dtype=torch.float16)
    with pytest.raises(TypeError, match="packed"):
        axr.quantize_keys(keys, BITS, 3, packed=torch.zeros(4, 12, dtype=torch.float32))
    with pytest.raises(TypeError, match="norms"):
        axr.quantize_keys(keys, BITS, 3, norms=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        axr.quantize_keys(keys, BITS, 3)


def test_score_outputs():
    q = torch.zeros(1, 4, 128)
    packed = torch.zeros(1, 1, 10, 12, dtype=torch.int32)
    norms = torch.zeros(1, 1, 10)
    with pytest.raises(TypeError, match="out"):
        axr.score(q, packed, norms, BITS, 3, out=torch.zeros(1, 4, 10, dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        axr.score(q, packed, norms, BITS, 3, out=torch.zeros(1, 4, 9))
    with pytest.raises(TypeError, match="packed"):
        axr.score(q, packed.float(), norms, BITS, 3)
    with pytest.raises(ValueError, match="GPU"):
        axr.score(q, packed, norms, BITS, 3)
    with pytest.raises(ValueError, match="shape"):
        axr.score_softmax(q, packed, norms, BITS, 3, lse=torch.zeros(1, 3))
    with pytest.raises(ValueError, match="shape"):
        axr.decode_step(q, torch.zeros(1, 1, 128), BITS, 3, packed, norms,
                        torch.zeros(1, dtype=torch.int32), out=torch.zeros(1, 4, 11))


def test_transform_output_shape():
    x = torch.zeros(3, 128)
    with pytest.raises(ValueError, match="shape"):
        axr.transform(x, BITS, out=torch.zeros(2, 128))
    with pytest.raises(TypeError, match="out"):
        axr.transform(x, BITS, out=torch.zeros(3, 128, dtype=torch.float64))
    quats = torch.zeros(32, 2, 4)
    with pytest.raises(ValueError, match="shape"):
        axr.transform_isoquant(x, quats, out=torch.zeros(3, 64))


def test_append_and_probe_arguments():
    packed = torch.zeros(2, 1, 8, 12, dtype=torch.int32)
    norms = torch.zeros(2, 1, 8)
    keys = torch.zeros(2, 1, 128)
    with pytest.raises(ValueError, match="pos"):
        axr.append_keys(keys, BITS, 3, packed, norms, torch.zeros(2, dtype=torch.int64))
    with pytest.raises(TypeError, match="norms"):
        axr.append_keys(keys, BITS, 3, packed, norms.double(), torch.zeros(2, dtype=torch.int32))
    buf = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="exceeds"):
        axr.probe_read_stream(buf, torch.zeros(1, dtype=torch.int32), nbytes=128)
    with pytest.raises(ValueError, match="sink"):
        axr.probe_read_stream(buf, torch.zeros(2, dtype=torch.uint8))
    with pytest.raises(ValueError, match="exceed"):
        axr.probe_read_write(buf, 65, buf, 16)
