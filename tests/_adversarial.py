"""Worst-case inputs for the score kernel's fixed-point table.

The read path (AXELRAM, Abstract: table lookup on read) sums table entries
q'_j c_k.  The kernel holds each coordinate term rounded to an integer
multiple of 2^-sh, with a per-head power of two chosen from the query so that
F = 2^sh sum_j |q'_j| max|c| lies just under [2^30, 2^31).  A score then
carries at most d/2 units (2^-sh) of table rounding, while the tolerance scale
||k|| sum_j |q'_j c_idx_j| is smallest, relative to F, when the key's indices
sit in the innermost cells.  The inputs built here drive that ratio to its
limit:

* one-hot queries q = alpha e_m: every |q'_j| equals alpha / sqrt(d), so
  every coordinate term of an index has the same magnitude (their roundings
  have the same size), and alpha puts F at the bottom of its range;
* unit keys whose transformed coordinates sit at the smallest positive
  centroid, signed like q' (every term positive, so the roundings add up),
  except one coordinate that carries the rest of the norm in the top cell;
* a spread of alphas per head group sweeps the rounded terms' fractional
  parts through [0, 1), so that some head rounds every term the same way by
  close to half a unit.

Built from the oracle's codebook and Hadamard matrix only.
"""

import functools

import numpy as np

from oracle import axelram as A
from workloads import sign_bits


@functools.lru_cache(maxsize=None)
def codebook(d, b):
    """The oracle's codebook, solved once per (d, b) here."""
    c, t = A.lloyd_max_codebook(d, b)
    c.setflags(write=False)
    t.setflags(write=False)
    return c, t

# The kernel's guard factor on the fixed-point full scale.
SCALE_GUARD = 1.0001


def one_hot_queries(d, b, G, rng, powers=(0,)):
    """Queries [G, d] (fp64, exactly representable in fp32 up to alpha's own
    rounding) q_g = alpha_g e_{m_g}.  alpha_g sqrt(d) max|c| times the guard
    factor is 2^k (1 + eps_g) with eps_g from 2e-6 to 1.2e-5, so the chosen
    full scale F is 2^30 (1 + eps_g) / 1.0001, the bottom of its range, while
    the terms' fractional parts sweep a full unit across the group."""
    c, _ = codebook(d, b)
    cmax = float(np.float32(c[-1]))
    q = np.zeros((G, d))
    ms = rng.integers(0, d, size=G)
    for g in range(G):
        k = powers[g % len(powers)]
        eps = 2e-6 + 1e-5 * g / max(G - 1, 1)
        alpha = 2.0 ** k * (1.0 + eps) / (np.sqrt(d) * cmax * SCALE_GUARD)
        q[g, ms[g]] = float(np.float32(alpha)) * (1.0 if rng.random() < 0.5 else -1.0)
    return q


def aligned_unit_y(qprime_g, b, spike, rng=None):
    """Transformed coordinates y (unit length) of a key aimed at the query
    transform qprime_g [d]: y_j = sign(q'_j) c_in for j != spike (c_in the
    smallest positive centroid), y_spike = sign(q'_spike) sqrt(1 - (d-1) c_in^2),
    which lies in the top cell."""
    d = qprime_g.shape[0]
    c, t = codebook(d, b)
    c_in = c[len(c) // 2]
    sg = np.where(qprime_g >= 0, 1.0, -1.0)
    y = sg * c_in
    top = np.sqrt(1.0 - (d - 1) * c_in ** 2)
    assert top > t[-1]
    y[spike] = sg[spike] * top
    return y


def keys_from_y(y, signs, norms):
    """Keys k = ||k|| D H y / sqrt(d) (the inverse of the write transform
    applied to unit y): [n, d] fp64."""
    d = y.shape[-1]
    h = A.sylvester_hadamard(d)
    return (np.asarray(norms)[:, None] * signs[None, :]) * (y @ h) / np.sqrt(d)


def worst_case_inputs(d, b, G, T, seed, powers=(0,)):
    """One KV head: queries [1, G, d] and keys [1, 1, T, d] (fp64), token t
    aimed at query head t % G with its spike at a random coordinate."""
    rng = np.random.default_rng(seed)
    bits = sign_bits(d)
    s = A.signs_from_bits(bits)
    q = one_hot_queries(d, b, G, rng, powers)
    qp = A.transform_queries(q[None], s)[0]
    ys = np.stack([aligned_unit_y(qp[t % G], b, int(rng.integers(0, d)))
                   for t in range(T)])
    norms = rng.uniform(0.5, 2.0, size=T)
    k = keys_from_y(ys, s, norms)
    return q[None], k[None, None], bits


def table_rounding_bound(d, b):
    """Largest table rounding of a score relative to ||k|| sum_j |q'_j c_idx_j|:
    d/2 units of 2^-sh against F >= 2^30 / 1.0001 units, with
    sum_j |q'_j c_idx_j| >= sum_j |q'_j| min|c| = F min|c| / max|c|."""
    c, _ = codebook(d, b)
    c_in, c_max = c[len(c) // 2], c[-1]
    return (d / 2) * SCALE_GUARD * (c_max / c_in) / 2.0 ** 30
