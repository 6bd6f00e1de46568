"""C-ABI checks that need no GPU: the library loads, exports what
include/axr.h declares, solves the codebook on the host, and rejects bad
arguments before any HIP call."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import lut_attention_scoring_amd as axr
from oracle import axelram as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000      # an aligned, never-dereferenced address
SIGNS = (ctypes.c_uint32 * 16)()


def declared_symbols():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            with open(os.path.join(ROOT, "include", fn)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            names |= set(re.findall(r"\b(axr_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert {"axr_codebook", "axr_quantize_keys", "axr_score", "axr_transform",
            "axr_last_error", "axr_version"} <= set(names)
    raw = ctypes.CDLL(axr.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name


def test_version():
    assert axr.version() >= 10000


@pytest.mark.parametrize("d", [1, 2, 64, 128, 256, 512])
@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_codebook_matches_oracle(d, b):
    c, t = axr.codebook(d, b)
    oc, ot = A.lloyd_max_codebook(d, b)
    sigma = 1.0 / math.sqrt(d)
    assert np.max(np.abs(c - oc)) <= 1e-12 * sigma
    assert np.max(np.abs(t - ot)) <= 1e-12 * sigma
    assert t[len(t) // 2] == 0.0
    np.testing.assert_array_equal(c, -c[::-1])


def _status(fn, *args):
    st = fn(*args)
    msg = axr.lib.axr_last_error().decode()
    return st, msg


def test_codebook_rejects_bad_arguments():
    c = (ctypes.c_double * 16)()
    t = (ctypes.c_double * 15)()
    assert _status(axr.lib.axr_codebook, 0, 3, c, t)[0] == axr.EINVAL
    assert _status(axr.lib.axr_codebook, 128, 5, c, t)[0] == axr.EINVAL
    assert _status(axr.lib.axr_codebook, 128, 0, c, t)[0] == axr.EINVAL
    st, msg = _status(axr.lib.axr_codebook, 128, 3, None, t)
    assert st == axr.EINVAL and "null" in msg


def _q(keys=FAKE, dtype=axr.F16, n=16, d=128, b=3, signs=SIGNS, packed=FAKE, norms=FAKE):
    return _status(axr.lib.axr_quantize_keys, keys, dtype, n, d, b, signs, packed, norms, None)


def test_quantize_validation():
    assert _q(d=100)[0] == axr.EUNSUPPORTED
    assert _q(d=64)[0] == axr.EUNSUPPORTED
    assert _q(b=1)[0] == axr.EUNSUPPORTED
    assert _q(b=5)[0] == axr.EUNSUPPORTED
    assert _q(dtype=9)[0] == axr.EUNSUPPORTED
    assert _q(n=-1)[0] == axr.EINVAL
    assert _q(signs=None)[0] == axr.EINVAL
    assert _q(keys=None)[0] == axr.EINVAL
    assert _q(packed=None)[0] == axr.EINVAL
    assert _q(norms=None)[0] == axr.EINVAL
    assert _q(keys=FAKE + 8)[0] == axr.EALIGN
    assert _q(packed=FAKE + 4)[0] == axr.EALIGN
    assert _q(norms=FAKE + 2)[0] == axr.EALIGN
    st, msg = _q(d=100)
    assert "d=100" in msg
    # n = 0 is a no-op that never touches the device, even with null buffers
    assert _q(n=0, keys=None, packed=None, norms=None)[0] == axr.OK
    assert axr.lib.axr_last_error().decode() == ""


def _s(q=FAKE, qdt=axr.F16, packed=FAKE, norms=FAKE, signs=SIGNS, B=2, Hq=8, Hkv=2, T=64,
       t_cap=64, d=128, b=3, scores=FAKE):
    return _status(axr.lib.axr_score, q, qdt, packed, norms, signs, B, Hq, Hkv, T, t_cap, d, b,
                   scores, None)


def test_score_validation():
    assert _s(d=96)[0] == axr.EUNSUPPORTED
    assert _s(b=7)[0] == axr.EUNSUPPORTED
    assert _s(qdt=5)[0] == axr.EUNSUPPORTED
    assert _s(Hq=6, Hkv=4)[0] == axr.EINVAL
    assert _s(Hkv=0)[0] == axr.EINVAL
    assert _s(B=-1)[0] == axr.EINVAL
    assert _s(T=-3)[0] == axr.EINVAL
    assert _s(t_cap=10, T=11)[0] == axr.EINVAL
    assert _s(Hq=130, Hkv=1)[0] == axr.EUNSUPPORTED
    assert _s(q=None)[0] == axr.EINVAL
    assert _s(scores=None)[0] == axr.EINVAL
    assert _s(signs=None)[0] == axr.EINVAL
    assert _s(q=FAKE + 4)[0] == axr.EALIGN
    assert _s(packed=FAKE + 8)[0] == axr.EALIGN
    assert _s(scores=FAKE + 1)[0] == axr.EALIGN
    assert _s(T=0, t_cap=0, q=None, packed=None, norms=None, scores=None)[0] == axr.OK
    assert _s(B=0, q=None, packed=None, norms=None, scores=None)[0] == axr.OK


def _qs(keys=FAKE, kdt=axr.F16, q=FAKE, qdt=axr.F16, signs=SIGNS, B=2, Hq=8, Hkv=2, T=64,
        d=128, b=3, packed=FAKE, norms=FAKE, scores=FAKE):
    return _status(axr.lib.axr_quantize_score, keys, kdt, q, qdt, signs, B, Hq, Hkv, T, d, b,
                   packed, norms, scores, None)


def test_quantize_score_validation():
    # shapes the one-launch path is not built for are rejected, not routed
    assert _qs(d=256)[0] == axr.EUNSUPPORTED
    assert _qs(b=4)[0] == axr.EUNSUPPORTED
    assert _qs(Hq=16, Hkv=2, b=2)[0] == axr.EUNSUPPORTED   # G = 8 only at b = 3
    assert _qs(Hq=12, Hkv=2)[0] == axr.EUNSUPPORTED        # G = 6: two head groups
    assert _qs(Hq=32, Hkv=2)[0] == axr.EUNSUPPORTED        # G = 16
    assert _qs(kdt=7)[0] == axr.EUNSUPPORTED
    assert _qs(qdt=7)[0] == axr.EUNSUPPORTED
    assert _qs(T=(1 << 23) + 1)[0] == axr.EUNSUPPORTED     # > 2 GiB of fp16 keys per row
    assert _qs(Hq=6, Hkv=4)[0] == axr.EINVAL
    assert _qs(B=-1)[0] == axr.EINVAL
    assert _qs(keys=None)[0] == axr.EINVAL
    assert _qs(scores=None)[0] == axr.EINVAL
    assert _qs(signs=None)[0] == axr.EINVAL
    assert _qs(keys=FAKE + 8)[0] == axr.EALIGN
    assert _qs(packed=FAKE + 4)[0] == axr.EALIGN
    assert _qs(norms=FAKE + 2)[0] == axr.EALIGN
    st, msg = _qs(b=4)
    assert "b=4" in msg
    assert _qs(T=0, keys=None, q=None, packed=None, norms=None, scores=None)[0] == axr.OK
    assert _qs(B=0, keys=None, q=None, packed=None, norms=None, scores=None)[0] == axr.OK


def test_probe_validation():
    # the measurement probes reject bad arguments before any HIP call
    f = axr.lib.axr_probe_lds_read
    assert f(0, FAKE, None) == -1
    assert f(65537, FAKE, None) == -1
    assert f(4, None, None) == -1
    assert f(4, FAKE + 2, None) == -1
    assert axr.lib.axr_probe_read_stream(FAKE, 24, FAKE, None) == -1        # not a multiple of 16
    assert axr.lib.axr_probe_read_write(FAKE, 16, FAKE + 1, 4, None) == -1  # misaligned output


def test_transform_validation():
    f = axr.lib.axr_transform
    assert _status(f, FAKE, axr.F32, 4, 48, SIGNS, 1, FAKE, None)[0] == axr.EUNSUPPORTED
    assert _status(f, FAKE, axr.F32, -4, 128, SIGNS, 1, FAKE, None)[0] == axr.EINVAL
    assert _status(f, FAKE, axr.F32, 4, 128, SIGNS, 1, None, None)[0] == axr.EINVAL
    assert _status(f, FAKE, axr.F32, 4, 128, SIGNS, 1, FAKE + 4, None)[0] == axr.EALIGN
    assert _status(f, None, axr.F32, 0, 128, SIGNS, 1, None, None)[0] == axr.OK


def test_sign_words_marshalling():
    rng = np.random.default_rng(0)
    for d in (128, 256, 512):
        bits = rng.integers(0, 2, d)
        words = axr.sign_words(bits)
        acc = sum(int(v) << j for j, v in enumerate(bits))
        assert [int(w) for w in words] == [(acc >> (32 * k)) & 0xFFFFFFFF for k in range(d // 32)]


def test_score_rejects_rows_beyond_32bit_offsets():
    # 2^31 bytes of d=128, b=3 records is 44.7M tokens per row
    st, msg = _s(T=45_000_000, t_cap=45_000_000)
    assert st == axr.EUNSUPPORTED and "2 GiB" in msg
    # the smallest record (d=128, b=2: 32 B) bounds eight heads' score rows
    st, msg = _s(T=67_108_864, t_cap=67_108_864, b=2, Hq=16, Hkv=2)
    assert st == axr.EUNSUPPORTED and "2 GiB" in msg


def _a(keys=FAKE, dtype=axr.F16, B=2, Hkv=4, d=128, b=3, signs=SIGNS, pos=FAKE, t_cap=64,
       packed=FAKE, norms=FAKE):
    return _status(axr.lib.axr_append_keys, keys, dtype, B, Hkv, d, b, signs, pos, t_cap, packed,
                   norms, None)


def test_append_validation():
    assert _a(d=48)[0] == axr.EUNSUPPORTED
    assert _a(b=1)[0] == axr.EUNSUPPORTED
    assert _a(dtype=7)[0] == axr.EUNSUPPORTED
    assert _a(B=-1)[0] == axr.EINVAL
    assert _a(Hkv=-2)[0] == axr.EINVAL
    assert _a(t_cap=0)[0] == axr.EINVAL
    assert _a(pos=None)[0] == axr.EINVAL
    assert _a(keys=None)[0] == axr.EINVAL
    assert _a(packed=None)[0] == axr.EINVAL
    assert _a(norms=None)[0] == axr.EINVAL
    assert _a(signs=None)[0] == axr.EINVAL
    assert _a(pos=FAKE + 2)[0] == axr.EALIGN
    assert _a(keys=FAKE + 4)[0] == axr.EALIGN
    assert _a(packed=FAKE + 8)[0] == axr.EALIGN
    st, msg = _a(B=65536, Hkv=65536)
    assert st == axr.EUNSUPPORTED and "2^31" in msg
    # nothing to append: no-op with null buffers
    assert _a(B=0, keys=None, pos=None, packed=None, norms=None)[0] == axr.OK
    assert _a(Hkv=0, keys=None, pos=None, packed=None, norms=None)[0] == axr.OK


def _r(lens=FAKE, **kw):
    args = dict(q=FAKE, qdt=axr.F16, packed=FAKE, norms=FAKE, signs=SIGNS, B=2, Hq=8, Hkv=2,
                T=64, t_cap=64, d=128, b=3, scores=FAKE)
    args.update(kw)
    a = args
    return _status(axr.lib.axr_score_ragged, a["q"], a["qdt"], a["packed"], a["norms"],
                   a["signs"], a["B"], a["Hq"], a["Hkv"], lens, a["T"], a["t_cap"], a["d"],
                   a["b"], a["scores"], None)


def test_score_ragged_validation():
    assert _r(lens=None)[0] == axr.EINVAL
    assert _r(lens=FAKE + 2)[0] == axr.EALIGN
    assert _r(Hq=6, Hkv=4)[0] == axr.EINVAL
    assert _r(t_cap=10, T=11)[0] == axr.EINVAL
    assert _r(b=9)[0] == axr.EUNSUPPORTED
    assert _r(q=None)[0] == axr.EINVAL
    assert _r(lens=None, B=0, q=None, packed=None, norms=None, scores=None)[0] == axr.OK
    assert _r(lens=None, T=0, t_cap=0, q=None, packed=None, norms=None, scores=None)[0] == axr.OK


def test_softmax_validation():
    n = ctypes.c_int64(-1)
    f = axr.lib.axr_score_softmax_workspace
    assert _status(f, 2, 8, 2, 64, 128, 3, ctypes.byref(n))[0] == axr.OK and n.value > 0
    assert _status(f, 2, 8, 2, 64, 128, 3, None)[0] == axr.EINVAL
    assert _status(f, 2, 6, 4, 64, 128, 3, ctypes.byref(n))[0] == axr.EINVAL
    assert _status(f, 0, 8, 2, 64, 128, 3, ctypes.byref(n))[0] == axr.OK and n.value == 0
    g = axr.lib.axr_score_softmax

    def sm(ws=FAKE, ws_bytes=1 << 20, scale=0.1, probs=FAKE, lse=None, lens=None):
        return _status(g, FAKE, axr.F16, FAKE, FAKE, SIGNS, 2, 8, 2, lens, 64, 64, 128, 3,
                       ctypes.c_float(scale), probs, lse, ws, ws_bytes, None)
    assert sm(ws=None)[0] == axr.EINVAL
    assert sm(ws_bytes=8)[0] == axr.EINVAL
    assert sm(scale=float("inf"))[0] == axr.EINVAL
    assert sm(probs=None)[0] == axr.EINVAL
    assert sm(ws=FAKE + 4)[0] == axr.EALIGN
    assert sm(lse=FAKE + 2)[0] == axr.EALIGN


def test_softmax_noalloc_validation():
    """The entry point without a workspace checks everything the workspace one
    does, and rejects sizes whose partials exceed its 1 MiB of library scratch
    before any device work (pointers here are never dereferenced)."""
    g = axr.lib.axr_score_softmax_noalloc

    def na(B=2, Hq=8, Hkv=2, T=64, q=FAKE, scale=0.1, probs=FAKE, lse=None):
        return _status(g, q, axr.F16, FAKE, FAKE, SIGNS, B, Hq, Hkv, None, T, T, 128, 3,
                       ctypes.c_float(scale), probs, lse, None)
    assert na(scale=float("nan"))[0] == axr.EINVAL
    assert na(q=None)[0] == axr.EINVAL
    assert na(probs=FAKE + 2)[0] == axr.EALIGN
    assert na(B=0, q=None, probs=None)[0] == axr.OK
    # 4096 x 64 rows x 1 tile x 8 B = 2 MiB of partials
    st, msg = na(B=4096, Hq=64, Hkv=1, T=1)
    assert st == axr.EUNSUPPORTED and "1048576 bytes of library scratch" in msg
    n = ctypes.c_int64(-1)
    assert _status(axr.lib.axr_score_softmax_workspace, 4096, 64, 1, 1, 128, 3,
                   ctypes.byref(n))[0] == axr.OK and n.value > 1 << 20


def test_sign_selection_validation():
    n = ctypes.c_int64(-1)
    f = axr.lib.axr_sign_selection_workspace
    assert _status(f, 8, 1, 16, 2, 2048, 128, 4, ctypes.byref(n))[0] == axr.OK
    assert n.value >= 8 * 16 * 2048 * 8
    assert _status(f, -1, 1, 16, 2, 2048, 128, 4, ctypes.byref(n))[0] == axr.EINVAL
    assert _status(f, 8, 1, 16, 2, 2048, 100, 4, ctypes.byref(n))[0] == axr.EUNSUPPORTED
    g = axr.lib.axr_sign_selection_errors
    cands = (ctypes.c_uint32 * 8)()

    def sel(keys=FAKE, dtype=axr.F16, C=2, cand=cands, errors=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return _status(g, keys, dtype, FAKE, axr.F16, 3, 1, 16, 2, 128, 128, 3, cand, C, errors,
                       ws, ws_bytes, None)
    assert sel(cand=None)[0] == axr.EINVAL
    assert sel(C=-1)[0] == axr.EINVAL
    assert sel(keys=None)[0] == axr.EINVAL
    assert sel(dtype=9)[0] == axr.EUNSUPPORTED
    assert sel(ws_bytes=16)[0] == axr.EINVAL
    assert sel(ws=FAKE + 16)[0] == axr.EALIGN
    assert sel(errors=FAKE + 4)[0] == axr.EALIGN
    assert sel(C=0, keys=None, cand=None, errors=None, ws=None)[0] == axr.OK


@pytest.mark.parametrize("seed", range(6))
def test_sign_selection_choose_matches_oracle(seed):
    """The library's choice rule (host) against the oracle's on random sums,
    with zero-reference samples (error zero and nonzero) and exact ties."""
    rng = np.random.default_rng(seed)
    C, S = int(rng.integers(1, 40)), int(rng.integers(1, 9))
    e = rng.uniform(0.0, 2.0, size=(C, S, 2)) ** 3
    e[rng.random((C, S)) < 0.1, 1] = 0.0
    e[rng.random((C, S)) < 0.1, 0] = 0.0
    if C > 2:
        e[C - 1] = e[C // 2]                       # a tie with an earlier candidate
    idx, obj = axr.sign_selection_choose(e)
    oidx, oobj = A.select_sign_pattern(e)
    assert idx == oidx
    assert np.array_equal(obj, oobj)


def test_sign_selection_choose_validation():
    f = axr.lib.axr_sign_selection_choose
    e = np.ones((3, 2, 2))
    dp = ctypes.POINTER(ctypes.c_double)
    idx = ctypes.c_int(-7)

    def ch(arr=e, C=3, S=2, index=ctypes.byref(idx)):
        ptr = None if arr is None else np.ascontiguousarray(arr).ctypes.data_as(dp)
        return _status(f, ptr, C, S, index, None)
    assert ch()[0] == axr.OK and idx.value == 0
    assert ch(C=0)[0] == axr.EINVAL
    assert ch(S=0)[0] == axr.EINVAL
    assert ch(arr=None)[0] == axr.EINVAL
    assert ch(index=None)[0] == axr.EINVAL
    for bad in (np.nan, -0.5):
        e2 = e.copy()
        e2[2, 1, 0] = bad
        idx.value = -7
        st, msg = ch(arr=e2)
        assert st == axr.EINVAL and "negative or NaN" in msg and idx.value == -7


def test_decode_step_validation():
    f = axr.lib.axr_decode_step

    def ds(q=FAKE, kdt=axr.F16, k=FAKE, pos=FAKE, packed=FAKE, norms=FAKE, scores=FAKE, B=2,
           T=64, t_cap=64):
        return _status(f, q, axr.F16, k, kdt, SIGNS, pos, B, 8, 2, T, t_cap, 128, 3, packed, norms,
                       scores, None)
    assert ds(kdt=7)[0] == axr.EUNSUPPORTED
    assert ds(k=None)[0] == axr.EINVAL
    assert ds(pos=None)[0] == axr.EINVAL
    assert ds(packed=None)[0] == axr.EINVAL
    assert ds(t_cap=10)[0] == axr.EINVAL
    assert ds(k=FAKE + 2)[0] == axr.EALIGN
    assert ds(packed=FAKE + 8)[0] == axr.EALIGN
    assert ds(B=0, q=None, k=None, pos=None, packed=None, norms=None, scores=None)[0] == axr.OK


def test_codebook_cache_and_errors_are_thread_safe():
    """Concurrent first solves of the same (d, b) keys agree with a serial
    solve, and each thread reads back its own last-error message."""
    import threading

    keys = [(d, b) for d in range(3, 60, 4) for b in (1, 2, 3, 4)]
    results = {}
    errors = []
    barrier = threading.Barrier(8)

    def worker(tid):
        barrier.wait()
        mine = {}
        order = keys[tid:] + keys[:tid]
        for d, b in order:
            mine[(d, b)] = axr.codebook(d, b)
            bad = -(1000 + 8 * d + tid)
            st = axr.lib.axr_codebook(bad, b, None, None)
            msg = axr.lib.axr_last_error().decode()
            if st != axr.EINVAL or f"d={bad}" not in msg:
                errors.append((tid, st, msg))
        results[tid] = mine

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
    for (d, b) in keys:
        ref_c, ref_t = axr.codebook(d, b)
        for tid in range(8):
            c, t = results[tid][(d, b)]
            np.testing.assert_array_equal(c, ref_c)
            np.testing.assert_array_equal(t, ref_t)
    oc, ot = A.lloyd_max_codebook(7, 3)
    c, t = axr.codebook(7, 3)
    assert np.max(np.abs(c - oc)) <= 1e-12 / math.sqrt(7)
