"""Parity criteria between the HIP path and the fp64 oracle.

Indices: bit-exact except coordinates whose oracle value (unit-normalised key,
after the transform) lies within 1e-6 of a codebook threshold; those may land
in the neighbouring cell, and there may be at most 1e-4 of all coordinates of
them, or 2 where that is fewer (the share of coordinates inside the window is
itself ~1e-4 at b = 3, so on a sample of a few thousand coordinates the
fraction alone would forbid a single legitimate flip).  Scores: given the GPU's own indices, within 1e-5 of
||k|| * sum_j |LUT[j][idx_j]| (the scale of any summation order's rounding).
Transform: within 1e-5 absolute on unit keys, 1e-5 * ||q|| on queries.
"""

import numpy as np
import torch

from oracle import axelram as A

BOUNDARY_WINDOW = 1e-6
MAX_MISMATCH_FRACTION = 1e-4
MIN_MISMATCH_ALLOWANCE = 2
SCORE_RTOL = 1e-5
TRANSFORM_ATOL = 1e-5
NORM_RTOL = 1e-5


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def words_u32(packed: torch.Tensor) -> np.ndarray:
    return packed.detach().cpu().numpy().view(np.uint32)


def assert_indices(gpu_idx, ora_idx, ora_y, thresholds, label=""):
    gpu_idx = np.asarray(gpu_idx)
    ora_idx = np.asarray(ora_idx)
    bad = gpu_idx != ora_idx
    nbad = int(bad.sum())
    total = ora_idx.size
    if nbad:
        yb = np.asarray(ora_y)[bad]
        dist = np.min(np.abs(yb[:, None] - np.asarray(thresholds)[None, :]), axis=1)
        assert float(dist.max()) < BOUNDARY_WINDOW, \
            f"{label}: index mismatch {dist.max():.3e} away from any threshold"
        assert np.all(np.abs(gpu_idx[bad] - ora_idx[bad]) == 1), f"{label}: non-adjacent cell"
    assert nbad <= max(MAX_MISMATCH_FRACTION * total, MIN_MISMATCH_ALLOWANCE), \
        f"{label}: {nbad} of {total} indices differ"
    return nbad, total


# Plain relative score errors |s_gpu - s_ref| / |s_ref| over the scores with
# |s_ref| >= 1e-2 of the checked set's rms, reported beside the
# condition-scaled bound (which is what is asserted): (label, scores counted,
# worst condition-scaled error, worst plain relative error).
PLAIN_REPORT = []


def plain_relative_error(got, ref):
    """Largest |got - ref| / |ref| over |ref| >= 1e-2 rms(ref), and how many
    scores that covers."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0, 0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    big = np.abs(ref) >= 1e-2 * rms
    if rms == 0.0 or not big.any():
        return 0.0, 0
    return float(np.max(np.abs(got[big] - ref[big]) / np.abs(ref[big]))), int(big.sum())


def assert_scores(gpu_scores, qprime, idx, norms, centroids, label=""):
    """gpu_scores [B, Hq, T]; idx [B, Hkv, T, d] (the GPU's); norms [B, Hkv, T] (fp64)."""
    ref = A.lut_scores(qprime, idx, norms, centroids)
    cond = A.score_condition(qprime, idx, norms, centroids)
    got = np.asarray(gpu_scores, np.float64)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(cond, 1e-300))) if err.size else 0.0
    plain, counted = plain_relative_error(got, ref)
    PLAIN_REPORT.append((label, counted, worst, plain))
    assert np.all(err <= SCORE_RTOL * cond), f"{label}: score error {worst:.3e} of condition"
    return worst


def assert_norms(gpu_norms, ora_norms, label=""):
    g = np.asarray(gpu_norms, np.float64)
    o = np.asarray(ora_norms, np.float64)
    assert np.all(np.abs(g - o) <= NORM_RTOL * o), f"{label}: norm mismatch"


def softmax_bounds(ref_scores, cond, scale, n_tok):
    """Per-element bound on |log p_gpu - log p_ref| for one row's first n_tok
    tokens (p_ref from the exact scores of the GPU's indices).  The score
    error bound eps_t = SCORE_RTOL * cond_t moves log p_t by at most
    scale * (eps_t + max eps) (the log-sum-exp moves by at most scale * max
    eps); fp32 adds rounding of the exponent argument and of the exponentials,
    the split sums and the division: 2^-22 (|scale s_t - M| + 2 |M|) + 8e-6."""
    x = scale * np.asarray(ref_scores, np.float64)[..., :n_tok]
    eps = SCORE_RTOL * np.asarray(cond, np.float64)[..., :n_tok]
    m = x.max(axis=-1, keepdims=True)
    bound = scale * (eps + eps.max(axis=-1, keepdims=True)) + 2.0 ** -22 * (
        np.abs(x - m) + 2 * np.abs(m)) + 8e-6
    lse_bound = (scale * eps.max(axis=-1) + 2.0 ** -22 * np.abs(m[..., 0]) * 2 + 8e-6)
    return bound, lse_bound


def assert_softmax(gpu_probs, gpu_lse, ref_scores, cond, scale, n_tok, label=""):
    """gpu_probs [Hq, T] and gpu_lse [Hq] of one batch row against the oracle
    softmax of ref_scores [Hq, T] (exact scores of the GPU's indices)."""
    p_ref, lse_ref = A.softmax_probs(np.asarray(ref_scores)[None], [n_tok], scale)
    p_ref, lse_ref = p_ref[0, :, :n_tok], lse_ref[0]
    bound, lse_bound = softmax_bounds(ref_scores, cond, scale, n_tok)
    got = np.asarray(gpu_probs, np.float64)[:, :n_tok]
    # |log p_gpu - log p_ref| <= bound, taken in the log domain (log p_ref =
    # scale s - lse never underflows), with probabilities below fp32's normal
    # range allowed to flush
    log_ref = scale * np.asarray(ref_scores, np.float64)[:, :n_tok] - lse_ref[:, None]
    hi = np.exp(np.minimum(log_ref + bound, 0.0))
    lo = np.exp(log_ref - bound)
    ok = (got <= hi + 2.0 ** -126) & (got >= lo - 2.0 ** -126)
    err = np.abs(got - p_ref)
    assert np.all(ok), f"{label}: probability error {float((err / np.maximum(p_ref, 1e-300)).max()):.3e}"
    lerr = np.abs(np.asarray(gpu_lse, np.float64) - lse_ref)
    assert np.all(lerr <= lse_bound), f"{label}: lse error {float(lerr.max()):.3e}"
