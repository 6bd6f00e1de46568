"""Plain, slow, fp64 CPU oracle of the AXELRAM write and read paths.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code, tables or constants with the
HIP library; it receives the same seeded inputs and nothing else.

Source: "AXELRAM: Quantize Once, Never Dequantize" (arXiv 2604.02638),
Abstract.  The abstract fixes: an orthogonal transform on write that makes each
coordinate of a (unit) key approximately N(0, 1/d); a design-time codebook that
is the optimal scalar quantizer for that density and depends only on (d, b); a
table lookup on read with no inverse transform; and a seeded sign pattern.
Where the abstract is silent this module takes the plainest reading:

* the key is normalised to unit length and its Euclidean norm is stored
  (otherwise a per-coordinate N(0, 1/d) law cannot hold for arbitrary keys);
* the orthogonal transform is  y = H_d (s * x) / sqrt(d)  with s in {+1,-1}^d
  the sign pattern and H_d the Sylvester-ordered Walsh-Hadamard matrix
  H_d[i, j] = (-1)^popcount(i & j), signs applied first;
* the optimal quantizer is the Lloyd-Max quantizer (centroid + midpoint
  conditions) for N(0, 1/d); the Code-with-Papers record of the paper's
  repository lists a Lloyd-Max solver next to a target-pdf and a
  conditional-mean routine, which is the construction used here;
* index of a coordinate = number of thresholds strictly below it (a value
  equal to a threshold takes the lower cell);
* the read-path table for query q is LUT[j][c] = q'_j * c_c with
  q' = H_d (s * q) / sqrt(d) (queries are not normalised) and the score of
  key k is ||k|| * sum_j LUT[j][idx_j];
* a query head h reads KV head h // G where G = Hq / Hkv;
* the b-bit indices of one key are stored as a little-endian bit stream:
  bit r of idx_j is bit (j*b + r) of the key's record, record bit m is bit
  m % 32 of 32-bit word m // 32.

Every routine below is the definition written out with numpy in float64: the
Hadamard transform is the dense matrix product (no butterflies), the quantizer
is a comparison count, the score is a gather and a sum.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "gaussian_cell_mass",
    "gaussian_cell_mean",
    "lloyd_max_codebook",
    "codebook_distortion",
    "sylvester_hadamard",
    "signs_from_bits",
    "key_norms",
    "rotate",
    "transform_keys",
    "transform_queries",
    "quantize",
    "pack_indices",
    "unpack_indices",
    "build_lut",
    "lut_scores",
    "score_condition",
    "write_path",
    "read_path",
    "dequantize_then_dot",
    "multiplications_per_query",
    "append_keys",
    "read_path_ragged",
    "softmax_probs",
    "dense_scores",
    "sign_selection_errors",
    "select_sign_pattern",
    "quaternion_multiply",
    "quaternion_conjugate",
    "isoquant_rotate",
    "isoquant_unrotate",
    "isoquant_write_path",
    "reconstruction_mse",
    "rotation_fmas",
]

_SQRT2 = math.sqrt(2.0)


# ---------------------------------------------------------------------------
# Design-time codebook: Lloyd-Max quantizer for N(0, sigma^2), sigma^2 = 1/d.
# ---------------------------------------------------------------------------

def _phi(z: float) -> float:
    """Standard normal density."""
    if math.isinf(z):
        return 0.0
    return math.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def gaussian_cell_mass(lo: float, hi: float) -> float:
    """P(lo < Z <= hi) for Z ~ N(0, 1), written to avoid cancellation in the
    tails (erfc on the side away from zero)."""
    if lo >= 0.0:
        return 0.5 * (math.erfc(lo / _SQRT2) - math.erfc(hi / _SQRT2))
    if hi <= 0.0:
        return 0.5 * (math.erfc(-hi / _SQRT2) - math.erfc(-lo / _SQRT2))
    return 0.5 * (math.erf(hi / _SQRT2) - math.erf(lo / _SQRT2))


def gaussian_cell_mean(lo: float, hi: float) -> float:
    """E[Z | lo < Z <= hi] for Z ~ N(0, 1): (phi(lo) - phi(hi)) / mass."""
    return (_phi(lo) - _phi(hi)) / gaussian_cell_mass(lo, hi)


def lloyd_max_codebook(d: int, b: int, max_iter: int = 200000):
    """Lloyd-Max quantizer with 2^b levels for the density N(0, 1/d).

    AXELRAM (arXiv 2604.02638), Abstract: the optimal quantizer depends only
    on the dimension d and the bit width b.  The two optimality conditions
    (Lloyd 1982, Max 1960) are iterated to their fixed point:
      thresholds  t_i = (c_i + c_{i+1}) / 2                (midpoint)
      centroids   c_i = E[X | t_{i-1} < X <= t_i]           (centroid)
    with t_{-1} = -inf and t_{2^b - 1} = +inf.  The Gaussian is log-concave,
    so the fixed point is unique and plain iteration converges to it.

    Returns (centroids[2^b], thresholds[2^b - 1]) as ascending float64 arrays.
    """
    if d < 1 or b < 1:
        raise ValueError("d and b must be positive")
    sigma = 1.0 / math.sqrt(d)
    levels = 1 << b
    # Start from evenly spaced points on [-2 sigma, 2 sigma]; the fixed point
    # does not depend on the start.
    c = np.array([sigma * (-2.0 + 4.0 * (i + 0.5) / levels) for i in range(levels)],
                 dtype=np.float64)
    for _ in range(max_iter):
        t = 0.5 * (c[:-1] + c[1:])
        edges = [-math.inf] + [float(v) for v in t] + [math.inf]
        new = np.array([sigma * gaussian_cell_mean(edges[i] / sigma, edges[i + 1] / sigma)
                        for i in range(levels)], dtype=np.float64)
        delta = float(np.max(np.abs(new - c)))
        c = new
        if delta <= 1e-17 * sigma:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t


def codebook_distortion(d: int, centroids, thresholds) -> float:
    """Mean squared error E[(X - Q(X))^2] of the quantizer for X ~ N(0, 1/d),
    evaluated in closed form cell by cell:
    E[(X-c)^2 ; cell] = E[X^2 ; cell] - 2c E[X ; cell] + c^2 P(cell)."""
    sigma = 1.0 / math.sqrt(d)
    edges = [-math.inf] + [float(v) / sigma for v in thresholds] + [math.inf]
    total = 0.0
    for i, cval in enumerate(centroids):
        lo, hi = edges[i], edges[i + 1]
        mass = gaussian_cell_mass(lo, hi)
        first = _phi(lo) - _phi(hi)                      # E[Z ; cell]
        lo_t = 0.0 if math.isinf(lo) else lo * _phi(lo)
        hi_t = 0.0 if math.isinf(hi) else hi * _phi(hi)
        second = mass + lo_t - hi_t                      # E[Z^2 ; cell]
        cz = float(cval) / sigma
        total += second - 2.0 * cz * first + cz * cz * mass
    return total * sigma * sigma


# ---------------------------------------------------------------------------
# Orthogonal transform: sign pattern, then normalised Walsh-Hadamard.
# ---------------------------------------------------------------------------

def sylvester_hadamard(d: int) -> np.ndarray:
    """Dense H_d with H_d[i, j] = (-1)^popcount(i & j) (natural order)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d, dtype=np.int64)
    anded = i[:, None] & i[None, :]
    parity = np.zeros_like(anded)
    while np.any(anded):
        parity ^= anded & 1
        anded >>= 1
    return np.where(parity == 0, 1.0, -1.0)


def signs_from_bits(bits) -> np.ndarray:
    """Sign pattern s_j = -1 where bit j is set, +1 otherwise."""
    bits = np.asarray(bits)
    return np.where(bits.astype(np.int64) != 0, -1.0, 1.0)


def key_norms(keys) -> np.ndarray:
    """Euclidean norm of each key (last axis), in float64."""
    k = np.asarray(keys, dtype=np.float64)
    return np.sqrt(np.sum(k * k, axis=-1))


def rotate(x, signs) -> np.ndarray:
    """y = H_d (s * x) / sqrt(d) along the last axis (no normalisation)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = sylvester_hadamard(d)
    return ((x * np.asarray(signs, dtype=np.float64)) @ h.T) / math.sqrt(d)


def transform_keys(keys, signs):
    """Write-path transform: unit-normalise each key, then rotate.

    Returns (y, norms).  A zero key keeps norm 0 and maps to y = 0.
    """
    k = np.asarray(keys, dtype=np.float64)
    norms = key_norms(k)
    safe = np.where(norms > 0.0, norms, 1.0)
    unit = np.where(norms[..., None] > 0.0, k / safe[..., None], 0.0)
    return rotate(unit, signs), norms


def transform_queries(q, signs) -> np.ndarray:
    """Read-path query transform q' = H_d (s * q) / sqrt(d); no normalisation."""
    return rotate(q, signs)


# ---------------------------------------------------------------------------
# Scalar quantization and the packed index record.
# ---------------------------------------------------------------------------

def quantize(y, thresholds) -> np.ndarray:
    """idx = number of thresholds strictly below y (ties take the lower cell)."""
    y = np.asarray(y, dtype=np.float64)
    t = np.asarray(thresholds, dtype=np.float64)
    return np.sum(y[..., None] > t, axis=-1).astype(np.int64)


def pack_indices(idx, b: int) -> np.ndarray:
    """Little-endian bit stream of b-bit fields, returned as uint32 words.

    idx: int array [..., d] with values in [0, 2^b).  Output [..., d*b/32].
    """
    idx = np.asarray(idx, dtype=np.int64)
    d = idx.shape[-1]
    if (d * b) % 32:
        raise ValueError("d*b must be a multiple of 32")
    bits = ((idx[..., :, None] >> np.arange(b)) & 1).astype(np.uint8)   # [..., d, b]
    bits = bits.reshape(idx.shape[:-1] + (d * b,))                        # record bit j*b+r
    as_bytes = np.packbits(bits, axis=-1, bitorder="little")              # [..., d*b/8]
    return as_bytes.view("<u4").reshape(idx.shape[:-1] + (d * b // 32,)).astype(np.uint32)


def unpack_indices(words, d: int, b: int) -> np.ndarray:
    """Inverse of pack_indices."""
    w = np.ascontiguousarray(np.asarray(words, dtype="<u4"))
    as_bytes = w.view(np.uint8).reshape(w.shape[:-1] + (w.shape[-1] * 4,))
    bits = np.unpackbits(as_bytes, axis=-1, bitorder="little")[..., : d * b]
    bits = bits.reshape(w.shape[:-1] + (d, b)).astype(np.int64)
    return np.sum(bits << np.arange(b), axis=-1)


# ---------------------------------------------------------------------------
# Read path: per-query table and table-lookup accumulation.
# ---------------------------------------------------------------------------

def build_lut(qprime, centroids) -> np.ndarray:
    """LUT[..., j, c] = q'_j * c_c."""
    return np.asarray(qprime, dtype=np.float64)[..., :, None] * np.asarray(centroids, np.float64)


def _gather(lut_h, idx_h):
    # lut_h [d, L], idx_h [T, d] -> LUT[j, idx[t, j]] as [T, d]
    d = lut_h.shape[0]
    return lut_h[np.arange(d)[None, :], idx_h]


def lut_scores(qprime, idx, norms, centroids) -> np.ndarray:
    """Scores from indices: s[b, h, t] = ||k_t|| * sum_j LUT_h[j, idx[b, h//G, t, j]].

    qprime [B, Hq, d]; idx [B, Hkv, T, d]; norms [B, Hkv, T].  Returns [B, Hq, T].
    """
    qprime = np.asarray(qprime, dtype=np.float64)
    idx = np.asarray(idx)
    norms = np.asarray(norms, dtype=np.float64)
    nb, hq, _ = qprime.shape
    hkv, t = idx.shape[1], idx.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    lut = build_lut(qprime, centroids)
    out = np.empty((nb, hq, t), dtype=np.float64)
    for bi in range(nb):
        for h in range(hq):
            kv = h // g
            out[bi, h] = norms[bi, kv] * np.sum(_gather(lut[bi, h], idx[bi, kv]), axis=-1)
    return out


def score_condition(qprime, idx, norms, centroids) -> np.ndarray:
    """||k_t|| * sum_j |LUT_h[j, idx_j]|: the scale against which the rounding
    error of any summation order of the score is measured."""
    qprime = np.asarray(qprime, dtype=np.float64)
    norms = np.asarray(norms, dtype=np.float64)
    nb, hq, _ = qprime.shape
    hkv, t = idx.shape[1], idx.shape[2]
    g = hq // hkv
    lut = np.abs(build_lut(qprime, centroids))
    out = np.empty((nb, hq, t), dtype=np.float64)
    for bi in range(nb):
        for h in range(hq):
            kv = h // g
            out[bi, h] = norms[bi, kv] * np.sum(_gather(lut[bi, h], idx[bi, kv]), axis=-1)
    return out


# ---------------------------------------------------------------------------
# Whole paths.
# ---------------------------------------------------------------------------

def write_path(keys, signs, b: int):
    """Quantize keys [..., d]: returns dict(y, norms, idx, packed)."""
    k = np.asarray(keys, dtype=np.float64)
    d = k.shape[-1]
    _, thresholds = lloyd_max_codebook(d, b)
    y, norms = transform_keys(k, signs)
    idx = quantize(y, thresholds)
    return {"y": y, "norms": norms, "idx": idx, "packed": pack_indices(idx, b)}


def read_path(q, packed, norms, signs, b: int):
    """Score queries [B, Hq, d] against packed keys [B, Hkv, T, d*b/32]."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    centroids, _ = lloyd_max_codebook(d, b)
    idx = unpack_indices(packed, d, b)
    qprime = transform_queries(q, signs)
    return lut_scores(qprime, idx, norms, centroids)


def append_keys(packed, norms, keys, pos, signs, b: int):
    """Decode-step write.  Each key is quantized once, when it is written
    (AXELRAM, Abstract): key (bi, h) of keys [B, Hkv, d] goes through
    write_path and its record and norm are stored at slot pos[bi] of the cache
    packed [B, Hkv, t_cap, W], norms [B, Hkv, t_cap].  A sequence whose slot
    lies outside [0, t_cap) is left as it was.  Returns new arrays."""
    out_p = np.array(packed, dtype=np.uint32, copy=True)
    out_n = np.array(norms, dtype=np.float64, copy=True)
    new = write_path(keys, signs, b)
    t_cap = out_p.shape[2]
    for bi, slot in enumerate(np.asarray(pos).tolist()):
        if 0 <= slot < t_cap:
            out_p[bi, :, slot] = new["packed"][bi]
            out_n[bi, :, slot] = new["norms"][bi]
    return out_p, out_n


def read_path_ragged(q, packed, norms, signs, b: int, lens, T: int):
    """read_path for sequences of different lengths: row bi is scored for
    t < min(max(lens[bi], 0), T) and holds NaN elsewhere.  A key's score does
    not depend on the other keys, so this is read_path restricted to each
    row's tokens."""
    full = read_path(q, np.asarray(packed)[:, :, :T], np.asarray(norms)[:, :, :T], signs, b)
    out = np.full(full.shape, np.nan)
    for bi, length in enumerate(np.asarray(lens).tolist()):
        n_tok = min(max(int(length), 0), T)
        out[bi, :, :n_tok] = full[bi, :, :n_tok]
    return out


def softmax_probs(scores, lens, scale: float):
    """Attention weights from scores [B, Hq, T]: for row bi and
    t < n = min(max(lens[bi], 0), T),
        probs = exp(scale * s - M) / L,  M = max scale * s,  L = sum exp(scale * s - M),
    and lse = M + log L.  Entries t >= n are NaN; an empty row has lse = -inf.
    (The usual normalisation of attention scores; the scores are the
    table-lookup scores of the read path.)"""
    s = np.asarray(scores, dtype=np.float64)
    nb, hq, T = s.shape
    probs = np.full(s.shape, np.nan)
    lse = np.full((nb, hq), -np.inf)
    for bi, length in enumerate(np.asarray(lens).tolist()):
        n_tok = min(max(int(length), 0), T)
        if n_tok == 0:
            continue
        x = scale * s[bi, :, :n_tok]
        m = x.max(axis=-1, keepdims=True)
        e = np.exp(x - m)
        total = e.sum(axis=-1, keepdims=True)
        probs[bi, :, :n_tok] = e / total
        lse[bi] = (m + np.log(total))[:, 0]
    return probs, lse


def dense_scores(q, keys) -> np.ndarray:
    """Exact scores q_h . k_t in float64 for q [B, Hq, d], keys [B, Hkv, T, d]
    (query head h reads KV head h // (Hq / Hkv))."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    nb, hq, _ = q.shape
    g = hq // k.shape[1]
    out = np.empty((nb, hq, k.shape[2]))
    for bi in range(nb):
        for h in range(hq):
            out[bi, h] = k[bi, h // g] @ q[bi, h]
    return out


def sign_selection_errors(keys, q, candidate_bits, b: int) -> np.ndarray:
    """Objective terms of the one-time sign-pattern selection (AXELRAM,
    Abstract: gradient-free, a few hundred candidates, a few calibration
    samples).  The page's objective is perplexity, which needs model weights;
    the stand-in measures how far the table scores are from the exact scores:
    for candidate c and calibration sample i,
        err[c, i] = sum (s_lut - s_exact)^2,   ref[c, i] = sum s_exact^2
    over every (batch, query head, token) of the sample.  keys
    [S, B, Hkv, T, d], q [S, B, Hq, d], candidate_bits [C, d].
    Returns [C, S, 2] (err, ref)."""
    keys = np.asarray(keys, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    out = np.empty((len(candidate_bits), keys.shape[0], 2))
    exact = [dense_scores(q[i], keys[i]) for i in range(keys.shape[0])]
    for c, bits in enumerate(candidate_bits):
        s = signs_from_bits(bits)
        for i in range(keys.shape[0]):
            w = write_path(keys[i], s, b)
            lut = read_path(q[i], w["packed"], w["norms"], s, b)
            out[c, i, 0] = np.sum((lut - exact[i]) ** 2)
            out[c, i, 1] = np.sum(exact[i] ** 2)
    return out


def select_sign_pattern(errors):
    """The candidate whose worst calibration sample has the smallest relative
    score error sqrt(err / ref); returns (index, objective per candidate).
    The first candidate wins a tie.  A sample whose exact scores are all zero
    (ref = 0, e.g. a zero query) has no relative error to measure: it counts
    0 when its table scores are zero too (err = 0) and +inf otherwise.
    Negative or NaN sums are rejected."""
    e = np.asarray(errors, dtype=np.float64)
    if e.ndim != 3 or e.shape[-1] != 2 or e.shape[0] < 1 or e.shape[1] < 1:
        raise ValueError("errors must be [C >= 1][S >= 1][2]")
    if not np.all(e >= 0.0):
        raise ValueError("error sums must be nonnegative numbers")
    err, ref = e[..., 0], e[..., 1]
    ratio = np.full(err.shape, np.inf)
    pos = ref > 0.0
    ratio[pos] = err[pos] / ref[pos]
    ratio[~pos & (err == 0.0)] = 0.0
    objective = np.sqrt(ratio).max(axis=1)
    return int(np.argmin(objective)), objective


# ---------------------------------------------------------------------------
# Comparison transform: block-wise quaternion rotations ("IsoQuant:
# Hardware-Aligned SO(4) Isoclinic Rotations for LLM KV Cache Compression",
# arXiv 2603.28430, Abstract).  Each block of 4 coordinates
# (v[4m], v[4m+1], v[4m+2], v[4m+3]) is the quaternion w + x i + y j + z k;
# IsoQuant-Full maps it to q_L v conj(q_R), IsoQuant-Fast to q_L v, with
# unit quaternions q_L, q_R per block.  Used with the same Lloyd-Max
# quantizer as the Walsh-Hadamard path.
# ---------------------------------------------------------------------------

def quaternion_multiply(a, b) -> np.ndarray:
    """Hamilton product of quaternions stored as (w, x, y, z) on the last
    axis, from i^2 = j^2 = k^2 = ijk = -1."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    aw, ax, ay, az = a[..., 0], a[..., 1], a[..., 2], a[..., 3]
    bw, bx, by, bz = b[..., 0], b[..., 1], b[..., 2], b[..., 3]
    return np.stack([aw * bw - ax * bx - ay * by - az * bz,
                     aw * bx + ax * bw + ay * bz - az * by,
                     aw * by - ax * bz + ay * bw + az * bx,
                     aw * bz + ax * by - ay * bx + az * bw], axis=-1)


def quaternion_conjugate(q) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    return q * np.array([1.0, -1.0, -1.0, -1.0])


def isoquant_rotate(x, q_left, q_right=None) -> np.ndarray:
    """Block rotation of x [..., d]: block m -> q_left[m] v conj(q_right[m])
    (IsoQuant-Full), or q_left[m] v when q_right is None (IsoQuant-Fast).
    q_left, q_right: [d/4, 4]."""
    x = np.asarray(x, dtype=np.float64)
    v = x.reshape(*x.shape[:-1], x.shape[-1] // 4, 4)
    t = quaternion_multiply(np.asarray(q_left, np.float64), v)
    if q_right is not None:
        t = quaternion_multiply(t, quaternion_conjugate(q_right))
    return t.reshape(x.shape)


def isoquant_unrotate(y, q_left, q_right=None) -> np.ndarray:
    """Inverse of isoquant_rotate for unit quaternions:
    conj(q_left) w q_right."""
    y = np.asarray(y, dtype=np.float64)
    w = y.reshape(*y.shape[:-1], y.shape[-1] // 4, 4)
    if q_right is not None:
        w = quaternion_multiply(w, np.asarray(q_right, np.float64))
    t = quaternion_multiply(quaternion_conjugate(q_left), w)
    return t.reshape(y.shape)


def isoquant_write_path(keys, q_left, q_right, b: int):
    """The write path with the block rotation in place of the Hadamard
    transform: unit-normalise, rotate, quantize with the Lloyd-Max codebook
    for N(0, 1/d), pack.  q_right None selects IsoQuant-Fast."""
    k = np.asarray(keys, dtype=np.float64)
    d = k.shape[-1]
    _, thresholds = lloyd_max_codebook(d, b)
    norms = key_norms(k)
    safe = np.where(norms > 0.0, norms, 1.0)
    y = isoquant_rotate(k / safe[..., None], q_left, q_right)
    y = np.where(norms[..., None] > 0.0, y, 0.0)
    idx = quantize(y, thresholds)
    return {"y": y, "norms": norms, "idx": idx, "packed": pack_indices(idx, b)}


def reconstruction_mse(keys, idx, centroids, unrotate) -> float:
    """Mean over keys of ||k/||k|| - T^-1(c[idx])||^2 (stage-1
    quantize-dequantize error on unit vectors); `unrotate` maps rotated
    coordinates back."""
    k = np.asarray(keys, dtype=np.float64)
    unit = k / key_norms(k)[..., None]
    rec = unrotate(np.asarray(centroids, np.float64)[np.asarray(idx)])
    return float(np.mean(np.sum((unit - rec) ** 2, axis=-1)))


def rotation_fmas(d: int, kind: str) -> int:
    """Multiply-adds of one forward rotation of a d-vector: a Hamilton product
    is 16; IsoQuant-Full uses two per block of 4, IsoQuant-Fast one, and the
    Walsh-Hadamard transform uses additions only."""
    if kind == "wht":
        return 0
    per_block = {"isoquant_full": 32, "isoquant_fast": 16}[kind]
    return per_block * (d // 4)


def dequantize_then_dot(q, idx, norms, signs, centroids) -> np.ndarray:
    """The same scores computed the long way, in the original key space:
    reconstruct k~ = ||k|| * T^T c[idx] (T = H_d diag(s) / sqrt(d)) and take
    q . k~.  Used only to check the table-lookup identity."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    h = sylvester_hadamard(d)
    s = np.asarray(signs, dtype=np.float64)
    chat = np.asarray(centroids, np.float64)[np.asarray(idx)]            # [B,Hkv,T,d]
    k_rec = (chat @ h) / math.sqrt(d) * s                                 # T^T c = D H c / sqrt(d)
    k_rec = k_rec * np.asarray(norms, np.float64)[..., None]
    nb, hq, _ = q.shape
    hkv = k_rec.shape[1]
    g = hq // hkv
    out = np.empty((nb, hq, k_rec.shape[2]), dtype=np.float64)
    for bi in range(nb):
        for hh in range(hq):
            out[bi, hh] = k_rec[bi, hh // g] @ q[bi, hh]
    return out


def multiplications_per_query(n_keys: int, d: int, b: int):
    """Multiplications needed to score one query against n_keys keys.

    Dense dot products cost n_keys * d.  The table path costs d * 2^b
    multiplications to fill the table plus one multiplication by the stored
    norm per key.  Returns (dense, table, ratio).
    """
    dense = n_keys * d
    table = d * (1 << b) + n_keys
    return dense, table, dense / table
