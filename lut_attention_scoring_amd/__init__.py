"""Python binding of libaxr (AXELRAM-style LUT attention scoring for MI355X).

Argument marshalling only: every step of the write and read paths runs in the
HIP kernels of libaxr.so, reached through the C ABI declared in include/axr.h.
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: importing this package fails if the library has not been built.

Method: "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638),
Abstract.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "AxrError", "LIB_PATH", "lib", "version", "codebook", "sign_words",
    "packed_words", "quantize_keys", "append_keys", "decode_step", "quantize_score", "score",
    "score_softmax",
    "score_softmax_noalloc",
    "transform", "sign_selection_errors", "sign_selection_choose", "select_sign_pattern",
    "quantize_keys_isoquant", "transform_isoquant",
    "probe_read_stream",
    "probe_read_write",
    "probe_lds_read",
    "F32", "F16", "BF16",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaxr.so")

F32, F16, BF16 = 0, 1, 2
_DTYPES = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

OK, EINVAL, EUNSUPPORTED, EALIGN, EHIP = 0, -1, -2, -3, -4


class AxrError(RuntimeError):
    """A libaxr call returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"axr status {status}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing; build it with `python lut_attention_scoring_amd/build.py`")
    so = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    dp = ctypes.POINTER(ctypes.c_double)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    so.axr_version.restype = i32
    so.axr_version.argtypes = []
    so.axr_last_error.restype = ctypes.c_char_p
    so.axr_last_error.argtypes = []
    so.axr_codebook.restype = i32
    so.axr_codebook.argtypes = [i32, i32, dp, dp]
    so.axr_quantize_keys.restype = i32
    so.axr_quantize_keys.argtypes = [vp, i32, i64, i32, i32, u32p, vp, vp, vp]
    so.axr_score.restype = i32
    so.axr_score.argtypes = [vp, i32, vp, vp, u32p, i32, i32, i32, i64, i64, i32, i32, vp, vp]
    i32p = ctypes.c_void_p
    so.axr_append_keys.restype = i32
    so.axr_append_keys.argtypes = [vp, i32, i32, i32, i32, i32, u32p, i32p, i64, vp, vp, vp]
    so.axr_score_ragged.restype = i32
    so.axr_score_ragged.argtypes = [vp, i32, vp, vp, u32p, i32, i32, i32, i32p, i64, i64, i32,
                                    i32, vp, vp]
    so.axr_score_softmax_workspace.restype = i32
    so.axr_score_softmax_workspace.argtypes = [i32, i32, i32, i64, i32, i32,
                                               ctypes.POINTER(ctypes.c_int64)]
    so.axr_score_softmax.restype = i32
    so.axr_score_softmax.argtypes = [vp, i32, vp, vp, u32p, i32, i32, i32, vp, i64, i64, i32,
                                     i32, ctypes.c_float, vp, vp, vp, i64, vp]
    so.axr_score_softmax_noalloc.restype = i32
    so.axr_score_softmax_noalloc.argtypes = [vp, i32, vp, vp, u32p, i32, i32, i32, vp, i64, i64,
                                             i32, i32, ctypes.c_float, vp, vp, vp]
    so.axr_sign_selection_workspace.restype = i32
    so.axr_sign_selection_workspace.argtypes = [i32, i32, i32, i32, i64, i32, i32,
                                                ctypes.POINTER(ctypes.c_int64)]
    so.axr_sign_selection_errors.restype = i32
    so.axr_sign_selection_errors.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i64, i32, i32,
                                             u32p, i32, vp, vp, i64, vp]
    so.axr_sign_selection_choose.restype = i32
    so.axr_sign_selection_choose.argtypes = [dp, i32, i32, ctypes.POINTER(ctypes.c_int), dp]
    so.axr_quantize_keys_isoquant.restype = i32
    so.axr_quantize_keys_isoquant.argtypes = [vp, i32, i64, i32, i32, vp, i32, vp, vp, vp]
    so.axr_transform_isoquant.restype = i32
    so.axr_transform_isoquant.argtypes = [vp, i32, i64, i32, vp, i32, i32, vp, vp]
    so.axr_decode_step.restype = i32
    so.axr_decode_step.argtypes = [vp, i32, vp, i32, u32p, vp, i32, i32, i32, i64, i64, i32, i32,
                                   vp, vp, vp, vp]
    so.axr_quantize_score.restype = i32
    so.axr_quantize_score.argtypes = [vp, i32, vp, i32, u32p, i32, i32, i32, i64, i32, i32, vp,
                                      vp, vp, vp]
    so.axr_transform.restype = i32
    so.axr_transform.argtypes = [vp, i32, i64, i32, u32p, i32, vp, vp]
    so.axr_probe_read_stream.restype = i32
    so.axr_probe_read_stream.argtypes = [vp, i64, vp, vp]
    so.axr_probe_read_write.restype = i32
    so.axr_probe_read_write.argtypes = [vp, i64, vp, i64, vp]
    so.axr_probe_lds_read.restype = i32
    so.axr_probe_lds_read.argtypes = [i32, vp, vp]
    return so


lib = _load()


def _check(status: int):
    if status != OK:
        raise AxrError(status, lib.axr_last_error().decode())


def version() -> int:
    return int(lib.axr_version())


def codebook(d: int, b: int):
    """Lloyd-Max centroids [2^b] and thresholds [2^b - 1] for N(0, 1/d) (host)."""
    c = (ctypes.c_double * (1 << b))()
    t = (ctypes.c_double * max(1, (1 << b) - 1))()
    _check(lib.axr_codebook(d, b, c, t))
    return np.array(c[:], dtype=np.float64), np.array(t[: (1 << b) - 1], dtype=np.float64)


def sign_words(bits) -> np.ndarray:
    """Sign pattern as uint32 words: bit j % 32 of word j // 32 is bits[j]."""
    bits = np.asarray(bits).astype(np.uint32).reshape(-1)
    if bits.size % 32:
        raise ValueError("sign pattern length must be a multiple of 32")
    shifts = np.arange(32, dtype=np.uint32)
    return np.bitwise_or.reduce(bits.reshape(-1, 32) << shifts, axis=1).astype(np.uint32)


def _words_ptr(words: np.ndarray):
    words = np.ascontiguousarray(words, dtype=np.uint32)
    return words, words.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _need_dtype(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _need_out(t: torch.Tensor, shape, dtype, name: str):
    _need_dtype(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_cuda(*tensors):
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("tensors must live on a GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def packed_words(d: int, b: int) -> int:
    return d * b // 32


def quantize_keys(keys: torch.Tensor, sign_bits, b: int, packed: torch.Tensor = None,
                  norms: torch.Tensor = None):
    """Write path: keys [..., d] -> (packed int32 [..., d*b/32], norms fp32 [...]).

    `packed` holds the uint32 words of the record, viewed as int32."""
    d = keys.shape[-1]
    lead = keys.shape[:-1]
    if packed is None:
        packed = torch.empty(*lead, packed_words(d, b), dtype=torch.int32, device=keys.device)
    if norms is None:
        norms = torch.empty(*lead, dtype=torch.float32, device=keys.device)
    _need_dtype(packed, torch.int32, "packed")
    _need_dtype(norms, torch.float32, "norms")
    _need_cuda(keys, packed, norms)
    n = keys.numel() // d if d else 0
    if packed.numel() != n * packed_words(d, b) or norms.numel() != n:
        raise ValueError("packed/norms sizes do not match keys")
    words, wp = _words_ptr(sign_words(sign_bits))
    _check(lib.axr_quantize_keys(keys.data_ptr(), _dtype_code(keys), n, d, b, wp,
                                 packed.data_ptr(), norms.data_ptr(), _stream(keys)))
    return packed, norms


def append_keys(keys: torch.Tensor, sign_bits, b: int, packed: torch.Tensor,
                norms: torch.Tensor, pos: torch.Tensor):
    """Decode-step write: keys [B, Hkv, d] quantized into slot pos[bi] (int32
    device tensor [B]) of the cache packed [B, Hkv, t_cap, W], norms
    [B, Hkv, t_cap].  Sequences whose pos is outside [0, t_cap) are skipped."""
    B, Hkv, d = keys.shape
    Bc, Hc, t_cap, W = packed.shape
    if (Bc, Hc) != (B, Hkv) or W != packed_words(d, b) or tuple(norms.shape) != (B, Hkv, t_cap):
        raise ValueError("keys, packed and norms shapes disagree")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B,):
        raise ValueError("pos must be an int32 tensor of shape [B]")
    _need_dtype(packed, torch.int32, "packed")
    _need_dtype(norms, torch.float32, "norms")
    _need_cuda(keys, packed, norms, pos)
    words, wp = _words_ptr(sign_words(sign_bits))
    _check(lib.axr_append_keys(keys.data_ptr(), _dtype_code(keys), B, Hkv, d, b, wp,
                               pos.data_ptr(), t_cap, packed.data_ptr(), norms.data_ptr(),
                               _stream(keys)))
    return packed, norms


def decode_step(q: torch.Tensor, k_new: torch.Tensor, sign_bits, b: int, packed: torch.Tensor,
                norms: torch.Tensor, pos: torch.Tensor, T: int = None, out: torch.Tensor = None):
    """One decode step in one launch: k_new [B, Hkv, d] quantized into slot
    pos[bi] of the cache and q [B, Hq, d] scored over t < pos[bi] + 1
    -> scores fp32 [B, Hq, T] (T defaults to t_cap).  A slot in [T, t_cap)
    is stored but not scored."""
    B, Hq, d = q.shape
    Bc, Hkv, t_cap, W = packed.shape
    if Bc != B or W != packed_words(d, b) or tuple(norms.shape) != (B, Hkv, t_cap):
        raise ValueError("q, packed and norms shapes disagree")
    if tuple(k_new.shape) != (B, Hkv, d):
        raise ValueError("k_new must be [B, Hkv, d]")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (B,):
        raise ValueError("pos must be an int32 tensor of shape [B]")
    T = t_cap if T is None else int(T)
    if out is None:
        out = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    _need_dtype(packed, torch.int32, "packed")
    _need_dtype(norms, torch.float32, "norms")
    _need_out(out, (B, Hq, T), torch.float32, "out")
    _need_cuda(q, k_new, packed, norms, pos, out)
    words, wp = _words_ptr(sign_words(sign_bits))
    _check(lib.axr_decode_step(q.data_ptr(), _dtype_code(q), k_new.data_ptr(),
                               _dtype_code(k_new), wp, pos.data_ptr(), B, Hq, Hkv, T, t_cap, d,
                               b, packed.data_ptr(), norms.data_ptr(), out.data_ptr(),
                               _stream(q)))
    return out


def quantize_score(keys: torch.Tensor, q: torch.Tensor, sign_bits, b: int,
                   packed: torch.Tensor = None, norms: torch.Tensor = None,
                   out: torch.Tensor = None):
    """Write and read path in one launch: keys [B, Hkv, T, d] and q [B, Hq, d]
    -> (packed int32 [B, Hkv, T, W], norms fp32 [B, Hkv, T], scores fp32
    [B, Hq, T]), the results of quantize_keys followed by score.  Built for
    d = 128, b = 2 or 3 with Hq / Hkv <= 4, and Hq / Hkv = 8 at b = 3."""
    B, Hkv, T, d = keys.shape
    Bq, Hq, dq = q.shape
    if (Bq, dq) != (B, d):
        raise ValueError("keys and q shapes disagree")
    if packed is None:
        packed = torch.empty(B, Hkv, T, packed_words(d, b), dtype=torch.int32, device=keys.device)
    if norms is None:
        norms = torch.empty(B, Hkv, T, dtype=torch.float32, device=keys.device)
    if out is None:
        out = torch.empty(B, Hq, T, dtype=torch.float32, device=keys.device)
    _need_out(packed, (B, Hkv, T, packed_words(d, b)), torch.int32, "packed")
    _need_out(norms, (B, Hkv, T), torch.float32, "norms")
    _need_out(out, (B, Hq, T), torch.float32, "out")
    _need_cuda(keys, q, packed, norms, out)
    words, wp = _words_ptr(sign_words(sign_bits))
    _check(lib.axr_quantize_score(keys.data_ptr(), _dtype_code(keys), q.data_ptr(),
                                  _dtype_code(q), wp, B, Hq, Hkv, T, d, b, packed.data_ptr(),
                                  norms.data_ptr(), out.data_ptr(), _stream(keys)))
    return packed, norms, out


def score(q: torch.Tensor, packed: torch.Tensor, norms: torch.Tensor, sign_bits, b: int,
          T: int = None, out: torch.Tensor = None, lens: torch.Tensor = None):
    """Read path: q [B, Hq, d], packed [B, Hkv, t_cap, W], norms [B, Hkv, t_cap]
    -> scores fp32 [B, Hq, T] (T defaults to t_cap).  With `lens` (int32
    device tensor [B]) row bi is scored only for t < lens[bi]; later entries
    of `out` are left as they were."""
    B, Hq, d = q.shape
    Bk, Hkv, t_cap, W = packed.shape
    if Bk != B or W != packed_words(d, b) or tuple(norms.shape) != (B, Hkv, t_cap):
        raise ValueError("q, packed and norms shapes disagree")
    T = t_cap if T is None else int(T)
    if out is None:
        out = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    _need_dtype(packed, torch.int32, "packed")
    _need_dtype(norms, torch.float32, "norms")
    _need_out(out, (B, Hq, T), torch.float32, "out")
    _need_cuda(q, packed, norms, out)
    words, wp = _words_ptr(sign_words(sign_bits))
    if lens is None:
        _check(lib.axr_score(q.data_ptr(), _dtype_code(q), packed.data_ptr(), norms.data_ptr(),
                             wp, B, Hq, Hkv, T, t_cap, d, b, out.data_ptr(), _stream(q)))
    else:
        if lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
            raise ValueError("lens must be an int32 tensor of shape [B]")
        _need_cuda(lens)
        _check(lib.axr_score_ragged(q.data_ptr(), _dtype_code(q), packed.data_ptr(),
                                    norms.data_ptr(), wp, B, Hq, Hkv, lens.data_ptr(), T, t_cap,
                                    d, b, out.data_ptr(), _stream(q)))
    return out


def score_softmax_workspace_bytes(B: int, Hq: int, Hkv: int, T: int, d: int, b: int) -> int:
    n = ctypes.c_int64(0)
    _check(lib.axr_score_softmax_workspace(B, Hq, Hkv, T, d, b, ctypes.byref(n)))
    return int(n.value)


def score_softmax(q: torch.Tensor, packed: torch.Tensor, norms: torch.Tensor, sign_bits,
                  b: int, scale: float = None, T: int = None, lens: torch.Tensor = None,
                  out: torch.Tensor = None, lse: torch.Tensor = None,
                  workspace: torch.Tensor = None):
    """Attention probabilities softmax(scale * scores) over each row's tokens
    t < lens[bi] (all T when lens is None); returns (probs [B, Hq, T], lse
    [B, Hq]).  scale defaults to 1/sqrt(d).  The workspace for the split-T
    partials is allocated here unless given."""
    B, Hq, d = q.shape
    Bk, Hkv, t_cap, W = packed.shape
    if Bk != B or W != packed_words(d, b) or tuple(norms.shape) != (B, Hkv, t_cap):
        raise ValueError("q, packed and norms shapes disagree")
    T = t_cap if T is None else int(T)
    scale = 1.0 / float(d) ** 0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    need = score_softmax_workspace_bytes(B, Hq, Hkv, T, d, b)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=q.device)
    _need_dtype(packed, torch.int32, "packed")
    _need_dtype(norms, torch.float32, "norms")
    _need_out(out, (B, Hq, T), torch.float32, "out")
    _need_out(lse, (B, Hq), torch.float32, "lse")
    _need_cuda(q, packed, norms, out, lse, workspace)
    if lens is not None:
        if lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
            raise ValueError("lens must be an int32 tensor of shape [B]")
        _need_cuda(lens)
    words, wp = _words_ptr(sign_words(sign_bits))
    _check(lib.axr_score_softmax(q.data_ptr(), _dtype_code(q), packed.data_ptr(),
                                 norms.data_ptr(), wp, B, Hq, Hkv,
                                 None if lens is None else lens.data_ptr(), T, t_cap, d, b,
                                 scale, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(q)))
    return out, lse


def score_softmax_noalloc(q: torch.Tensor, packed: torch.Tensor, norms: torch.Tensor,
                          sign_bits, b: int, out: torch.Tensor, lse: torch.Tensor,
                          scale: float = None, T: int = None, lens: torch.Tensor = None):
    """score_softmax with the split-T partials in the library's own device
    array (no allocation here or in the library): out [B, Hq, T] and lse
    [B, Hq] must be given.  Calls that overlap on one device race on that
    array."""
    B, Hq, d = q.shape
    Bk, Hkv, t_cap, W = packed.shape
    if Bk != B or W != packed_words(d, b) or tuple(norms.shape) != (B, Hkv, t_cap):
        raise ValueError("q, packed and norms shapes disagree")
    T = t_cap if T is None else int(T)
    scale = 1.0 / float(d) ** 0.5 if scale is None else float(scale)
    _need_dtype(packed, torch.int32, "packed")
    _need_dtype(norms, torch.float32, "norms")
    _need_out(out, (B, Hq, T), torch.float32, "out")
    _need_out(lse, (B, Hq), torch.float32, "lse")
    _need_cuda(q, packed, norms, out, lse)
    if lens is not None:
        if lens.dtype != torch.int32 or tuple(lens.shape) != (B,):
            raise ValueError("lens must be an int32 tensor of shape [B]")
        _need_cuda(lens)
    words, wp = _words_ptr(sign_words(sign_bits))
    _check(lib.axr_score_softmax_noalloc(q.data_ptr(), _dtype_code(q), packed.data_ptr(),
                                         norms.data_ptr(), wp, B, Hq, Hkv,
                                         None if lens is None else lens.data_ptr(), T, t_cap, d,
                                         b, scale, out.data_ptr(), lse.data_ptr(), _stream(q)))
    return out, lse


def sign_selection_errors(keys: torch.Tensor, q: torch.Tensor, candidate_bits, b: int):
    """Per-candidate, per-sample score errors of the sign-pattern selection:
    keys [S, B, Hkv, T, d], q [S, B, Hq, d], candidate_bits [C, d] (host)
    -> float64 device tensor [C, S, 2] of (sum (s_lut - s_exact)^2,
    sum s_exact^2)."""
    S, B, Hkv, T, d = keys.shape
    Sq, Bq, Hq, dq = q.shape
    if (Sq, Bq, dq) != (S, B, d):
        raise ValueError("keys and q shapes disagree")
    bits = np.asarray(candidate_bits).reshape(-1, d)
    C = bits.shape[0]
    words = np.ascontiguousarray(np.stack([sign_words(r) for r in bits]) if C else
                                 np.zeros((0, d // 32)), dtype=np.uint32)
    wp = words.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32))
    nbytes = ctypes.c_int64(0)
    _check(lib.axr_sign_selection_workspace(S, B, Hq, Hkv, T, d, b, ctypes.byref(nbytes)))
    ws = torch.empty(max(256, nbytes.value), dtype=torch.uint8, device=keys.device)
    errors = torch.zeros(C, S, 2, dtype=torch.float64, device=keys.device)
    _need_cuda(keys, q, errors, ws)
    _check(lib.axr_sign_selection_errors(keys.data_ptr(), _dtype_code(keys), q.data_ptr(),
                                         _dtype_code(q), S, B, Hq, Hkv, T, d, b, wp, C,
                                         errors.data_ptr(), ws.data_ptr(), ws.numel(),
                                         _stream(keys)))
    return errors


def sign_selection_choose(errors):
    """The library's choice rule on error sums [C, S, 2] (host array or
    tensor): returns (index, objective per candidate as a numpy array)."""
    if isinstance(errors, torch.Tensor):
        errors = errors.detach().cpu().numpy()
    e = np.ascontiguousarray(errors, dtype=np.float64)
    if e.ndim != 3 or e.shape[-1] != 2:
        raise ValueError("errors must have shape [C, S, 2]")
    C, S = e.shape[0], e.shape[1]
    objective = np.empty(max(C, 1), dtype=np.float64)
    index = ctypes.c_int(-1)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(lib.axr_sign_selection_choose(e.ctypes.data_as(dp), C, S, ctypes.byref(index),
                                         objective.ctypes.data_as(dp)))
    return int(index.value), objective[:C]


def select_sign_pattern(keys: torch.Tensor, q: torch.Tensor, candidate_bits, b: int):
    """Error sums of every candidate on the GPU, then the library's choice
    rule (the smallest worst-sample sqrt(err / ref)); returns (index,
    objective per candidate).  Synchronises with the device to read the
    sums."""
    return sign_selection_choose(sign_selection_errors(keys, q, candidate_bits, b))


def _quats(quats: torch.Tensor, d: int, device) -> torch.Tensor:
    if tuple(quats.shape) != (d // 4, 2, 4) or quats.dtype != torch.float32:
        raise ValueError("quats must be float32 [d/4, 2, 4]")
    if quats.device != device:
        raise ValueError("quats must live on the keys' device")
    return quats.contiguous()


def quantize_keys_isoquant(keys: torch.Tensor, quats: torch.Tensor, b: int, full: bool = True,
                           packed: torch.Tensor = None, norms: torch.Tensor = None):
    """Comparison write path with block-quaternion rotations (IsoQuant-Full or
    -Fast) instead of the Walsh-Hadamard transform; same codebook and layout."""
    d = keys.shape[-1]
    lead = keys.shape[:-1]
    quats = _quats(quats, d, keys.device)
    if packed is None:
        packed = torch.empty(*lead, packed_words(d, b), dtype=torch.int32, device=keys.device)
    if norms is None:
        norms = torch.empty(*lead, dtype=torch.float32, device=keys.device)
    _need_dtype(packed, torch.int32, "packed")
    _need_dtype(norms, torch.float32, "norms")
    _need_cuda(keys, packed, norms, quats)
    n = keys.numel() // d if d else 0
    if packed.numel() != n * packed_words(d, b) or norms.numel() != n:
        raise ValueError("packed/norms sizes do not match keys")
    _check(lib.axr_quantize_keys_isoquant(keys.data_ptr(), _dtype_code(keys), n, d, b,
                                          quats.data_ptr(), int(bool(full)), packed.data_ptr(),
                                          norms.data_ptr(), _stream(keys)))
    return packed, norms


def transform_isoquant(x: torch.Tensor, quats: torch.Tensor, full: bool = True,
                       normalize: bool = True, out: torch.Tensor = None):
    """Diagnostic: the block-quaternion rotation of each row (/ ||x|| if
    normalize), fp32 [..., d]."""
    d = x.shape[-1]
    quats = _quats(quats, d, x.device)
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _need_out(out, x.shape, torch.float32, "out")
    _need_cuda(x, out, quats)
    n = x.numel() // d if d else 0
    _check(lib.axr_transform_isoquant(x.data_ptr(), _dtype_code(x), n, d, quats.data_ptr(),
                                      int(bool(full)), int(bool(normalize)), out.data_ptr(),
                                      _stream(x)))
    return out


def transform(x: torch.Tensor, sign_bits, normalize: bool = True, out: torch.Tensor = None):
    """Diagnostic: y = H (s * x) / sqrt(d) (/ ||x|| if normalize), fp32 [..., d]."""
    d = x.shape[-1]
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    _need_out(out, x.shape, torch.float32, "out")
    _need_cuda(x, out)
    n = x.numel() // d if d else 0
    words, wp = _words_ptr(sign_words(sign_bits))
    _check(lib.axr_transform(x.data_ptr(), _dtype_code(x), n, d, wp, int(bool(normalize)),
                             out.data_ptr(), _stream(x)))
    return out


def probe_read_stream(buf: torch.Tensor, sink: torch.Tensor, nbytes: int = None):
    """Bandwidth probe (include/axr_probe.h): stream-read `nbytes` of `buf`."""
    nbytes = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if nbytes > buf.numel() * buf.element_size() or sink.numel() * sink.element_size() < 4:
        raise ValueError("probe size exceeds the buffer, or the sink is under 4 bytes")
    _need_cuda(buf, sink)
    if lib.axr_probe_read_stream(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(buf)) != 0:
        raise AxrError(EINVAL, "axr_probe_read_stream rejected its arguments")


def probe_read_write(src: torch.Tensor, in_bytes: int, dst: torch.Tensor, out_bytes: int):
    """Bandwidth probe: read `in_bytes` of `src`, write `out_bytes` of `dst`."""
    if (in_bytes > src.numel() * src.element_size()
            or out_bytes > dst.numel() * dst.element_size()):
        raise ValueError("probe sizes exceed the buffers")
    _need_cuda(src, dst)
    if lib.axr_probe_read_write(src.data_ptr(), int(in_bytes), dst.data_ptr(), int(out_bytes),
                                _stream(src)) != 0:
        raise AxrError(EINVAL, "axr_probe_read_write rejected its arguments")


def probe_lds_read(iters: int, out: torch.Tensor):
    """LDS probe (include/axr_probe.h): 256 blocks x 1024 threads read their
    128 KiB LDS array with 16-byte reads in the score kernel's table pattern,
    iters x 16 reads per thread; out is an int32 device tensor of >= 262144
    elements (checksums).  Returns the bytes read per CU."""
    if out.numel() * out.element_size() < 4 * 262144:
        raise ValueError("out must hold 262144 uint32 checksums")
    _need_cuda(out)
    if lib.axr_probe_lds_read(int(iters), out.data_ptr(), _stream(out)) != 0:
        raise AxrError(EINVAL, "axr_probe_lds_read rejected its arguments")
    return 1024 * 16 * int(iters) * 16
