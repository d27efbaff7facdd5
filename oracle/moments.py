"""Exact first and second moments of the three SANTA estimators (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The abstract claims the estimate is unbiased and that stratified and
systematic sampling reduce its variance.  These functions give the exact
per-coordinate mean and variance of the estimate o^ = (1/S) sum_k V[i_k] for
one query head, given the CDF F (F_{n-1} = 1) and the value rows V, so that
those claims, and Monte-Carlo runs of the sampler, can be checked without
sampling noise.  Textbook survey-sampling identities:

* i.i.d.: the S draws are independent with law p, so
  Var(o^_d) = (sum_j p_j V_jd^2 - o_d^2) / S.
* stratified: stratum k's point is uniform on [k/S, (k+1)/S); the key it
  selects has law p^(k)_j = S * |[F_{j-1}, F_j) intersect [k/S, (k+1)/S)|, and
  the strata are independent.
* systematic: with points (k + u) / S, key j receives
  g_j(u) - g_{j-1}(u) points where g_j(u) = ceil(S F_j - u); summing by parts,
  o^(u) = V_{n-1} + (1/S) sum_{j<n-1} g_j(u) (V_j - V_{j+1}), and
  g_j(u) = floor(S F_j) + [u < frac(S F_j)].  Integrating this step function
  of u over [0, 1) exactly gives the mean and variance.

Pinned in tests/test_oracle_moments.py by brute-force enumeration (i.i.d.) and
fine-grid integration over the uniforms (stratified, systematic), computed
with an independent linear-walk search.
"""

import numpy as np


def _pmf_from_cdf(F):
    F = np.asarray(F, dtype=np.float64)
    return np.diff(np.concatenate(([0.0], F)))


def iid_moments(F, V, S):
    """(mean, var) per coordinate for S i.i.d. draws from the law with CDF F."""
    p = _pmf_from_cdf(F)
    V = np.asarray(V, dtype=np.float64)
    mean = p @ V
    second = p @ (V * V)
    return mean, (second - mean * mean) / S


def stratum_laws(F, S):
    """Matrix P (S, n): P[k, j] = S * |[F_{j-1}, F_j) intersect [k/S, (k+1)/S)|."""
    F = np.asarray(F, dtype=np.float64)
    lo = np.concatenate(([0.0], F[:-1]))
    a = np.arange(S, dtype=np.float64)[:, None] / S
    b = (np.arange(S, dtype=np.float64)[:, None] + 1.0) / S
    overlap = np.minimum(F[None, :], b) - np.maximum(lo[None, :], a)
    return S * np.clip(overlap, 0.0, None)


def stratified_moments(F, V, S):
    """(mean, var) per coordinate for stratified sampling with S strata."""
    V = np.asarray(V, dtype=np.float64)
    P = stratum_laws(F, S)
    mean_k = P @ V
    second_k = P @ (V * V)
    mean = mean_k.sum(axis=0) / S
    var = (second_k - mean_k * mean_k).sum(axis=0) / (S * S)
    return mean, var


def systematic_moments(F, V, S):
    """(mean, var) per coordinate for systematic sampling with one offset."""
    F = np.asarray(F, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = len(F)
    if n == 1:
        return V[0].copy(), np.zeros(V.shape[1])
    x = S * F[:-1]
    m = np.floor(x)
    f = x - m  # o^(u) gains D_j / S while u < f_j
    D = V[:-1] - V[1:]
    base = V[-1] + (m @ D) / S  # value of o^ for u above every f_j
    # Sort the jump points; on (f_(r), f_(r+1)) the active set is the suffix.
    order = np.argsort(f, kind="stable")
    fs = f[order]
    Ds = D[order]
    suffix = np.cumsum(Ds[::-1], axis=0)[::-1]  # suffix[r] = sum_{i >= r} Ds[i]
    # interval r covers u in (fs[r-1], fs[r]) with active set order[r:]
    edges = np.concatenate(([0.0], fs))
    widths = np.diff(edges)  # widths[r] = fs[r] - fs[r-1]
    Y = suffix / S  # value above base on interval r
    # last interval (fs[-1], 1) has an empty active set: Y = 0
    mean_y = widths @ Y
    second_y = widths @ (Y * Y)
    mean = base + mean_y
    var = second_y - mean_y * mean_y
    return mean, var


def moments(mode, F, V, S):
    """Dispatch on the mode number (0 i.i.d., 1 stratified, 2 systematic)."""
    if mode == 0:
        return iid_moments(F, V, S)
    if mode == 1:
        return stratified_moments(F, V, S)
    if mode == 2:
        return systematic_moments(F, V, S)
    raise ValueError("unknown mode %r" % (mode,))
