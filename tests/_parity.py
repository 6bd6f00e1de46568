"""Parity criteria between the HIP path and the fp64 oracle.

Indices: bit-exact except coordinates whose oracle value (unit-normalised key,
after the transform) lies within 1e-6 of a codebook threshold; those may land
in the neighbouring cell, and there may be at most 1e-4 of all coordinates of
them.  Scores: given the GPU's own indices, within 1e-5 of
||k|| * sum_j |LUT[j][idx_j]| (the scale of any summation order's rounding).
Transform: within 1e-5 absolute on unit keys, 1e-5 * ||q|| on queries.
"""

import numpy as np
import torch

from oracle import axelram as A

BOUNDARY_WINDOW = 1e-6
MAX_MISMATCH_FRACTION = 1e-4
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
    assert nbad <= MAX_MISMATCH_FRACTION * total, f"{label}: {nbad} of {total} indices differ"
    return nbad, total


def assert_scores(gpu_scores, qprime, idx, norms, centroids, label=""):
    """gpu_scores [B, Hq, T]; idx [B, Hkv, T, d] (the GPU's); norms [B, Hkv, T] (fp64)."""
    ref = A.lut_scores(qprime, idx, norms, centroids)
    cond = A.score_condition(qprime, idx, norms, centroids)
    err = np.abs(np.asarray(gpu_scores, np.float64) - ref)
    worst = float(np.max(err / np.maximum(cond, 1e-300))) if err.size else 0.0
    assert np.all(err <= SCORE_RTOL * cond), f"{label}: score error {worst:.3e} of condition"
    return worst


def assert_norms(gpu_norms, ora_norms, label=""):
    g = np.asarray(gpu_norms, np.float64)
    o = np.asarray(ora_norms, np.float64)
    assert np.all(np.abs(g - o) <= NORM_RTOL * o), f"{label}: norm mismatch"
