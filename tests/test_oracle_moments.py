"""Pins for the exact-moment functions and for the abstract's claims (CPU).

* unbiasedness (the abstract's third sentence): the exact mean of every
  estimator equals dense attention;
* variance reduction (fourth sentence): stratified <= i.i.d. is a theorem for
  equal-probability strata; systematic <= stratified is not a theorem and is
  asserted only for the configured synthetic inputs.

The moment formulas themselves are pinned against brute-force enumeration and
fine-grid integration that use their own linear-walk search.
"""

import itertools

import numpy as np
import pytest

from oracle import moments as M
from oracle import santa as O
from stochastic_sparse_decode_amd import workloads as W


def _walk(cum_over_Z, t):
    j = 0
    while j < len(cum_over_Z) - 1 and cum_over_Z[j] <= t:
        j += 1
    return j


def _case(n, d, seed, spread=1.5):
    rng = np.random.default_rng(seed)
    s = spread * rng.standard_normal(n)
    V = rng.standard_normal((n, d))
    _, _, F = O.distribution(s)
    return s, V, F


def test_iid_moments_match_enumeration():
    s, V, F = _case(4, 3, 1)
    p = O.probabilities(s)
    S = 3
    mean = np.zeros(3)
    second = np.zeros(3)
    for tup in itertools.product(range(4), repeat=S):
        prob = np.prod(p[list(tup)])
        est = V[list(tup)].mean(axis=0)
        mean += prob * est
        second += prob * est ** 2
    m, v = M.iid_moments(F, V, S)
    np.testing.assert_allclose(m, mean, atol=1e-13)
    np.testing.assert_allclose(v, second - mean ** 2, atol=1e-13)


def test_stratified_moments_match_grid_integration():
    s, V, F = _case(7, 2, 2)
    S = 3
    grid = (np.arange(20000) + 0.5) / 20000  # midpoints in each stratum
    means, seconds = [], []
    for k in range(S):
        est = np.array([V[_walk(F, (k + u) / S)] for u in grid])
        means.append(est.mean(axis=0))
        seconds.append((est ** 2).mean(axis=0))
    means, seconds = np.array(means), np.array(seconds)
    mean = means.sum(axis=0) / S
    var = (seconds - means ** 2).sum(axis=0) / S ** 2
    m, v = M.stratified_moments(F, V, S)
    np.testing.assert_allclose(m, mean, atol=2e-4)
    np.testing.assert_allclose(v, var, atol=2e-4)


def test_systematic_moments_match_grid_integration():
    s, V, F = _case(9, 3, 3)
    S = 4
    grid = (np.arange(40000) + 0.5) / 40000
    est = np.array([np.mean([V[_walk(F, (k + u) / S)] for k in range(S)], axis=0) for u in grid])
    m, v = M.systematic_moments(F, V, S)
    np.testing.assert_allclose(m, est.mean(axis=0), atol=2e-4)
    np.testing.assert_allclose(v, est.var(axis=0), atol=2e-4)


@pytest.mark.parametrize("mode", O.MODES)
@pytest.mark.parametrize("n,S", [(1, 4), (5, 2), (100, 16), (1000, 128), (257, 1000)])
def test_every_mode_is_exactly_unbiased(mode, n, S):
    s, V, F = _case(n, 8, 10 + n, spread=2.0)
    dense = O.dense_head(s, V)
    m, v = M.moments(mode, F, V, S)
    np.testing.assert_allclose(m, dense, atol=1e-12, rtol=0)
    assert np.all(v >= -1e-12)


def test_systematic_with_S_equal_n_uniform_has_zero_variance():
    n = 64
    V = np.random.default_rng(4).standard_normal((n, 5))
    F = np.arange(1, n + 1) / n
    m, v = M.systematic_moments(F, V, n)
    np.testing.assert_allclose(m, V.mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(v, 0.0, atol=1e-14)


def test_stratified_never_exceeds_iid():
    """Law of total variance with equal-probability strata (a theorem)."""
    rng = np.random.default_rng(20)
    for trial in range(30):
        n = int(rng.integers(2, 300))
        S = int(rng.choice([2, 7, 32, 128]))
        s, V, F = _case(n, 4, 100 + trial, spread=float(rng.uniform(0.1, 4)))
        _, v_iid = M.iid_moments(F, V, S)
        _, v_str = M.stratified_moments(F, V, S)
        assert np.all(v_str <= v_iid * (1 + 1e-9) + 1e-15)


def _head_mse(wl, b, h, S, mode):
    G = wl.Hq // wl.Hkv
    n = int(wl.n_k[b])
    s = O.head_scores(wl.q[b, h].astype(np.float64), wl.K[b, h // G, :n].astype(np.float64), wl.scale)
    _, _, F = O.distribution(s)
    _, var = M.moments(mode, F, wl.V[b, h // G, :n].astype(np.float64), S)
    return var.sum()


@pytest.mark.parametrize("S", [16, 64])
def test_variance_ordering_on_tiny_config(S):
    wl = W.tiny()
    v = {mode: _head_mse(wl, 0, 0, S, mode) for mode in O.MODES}
    assert v[O.SYSTEMATIC] <= v[O.STRATIFIED] <= v[O.IID]


def test_variance_ordering_on_llama_shaped_heads():
    wl = W.llama(B=1, n_k=4096, seed=21)
    for h in (0, 5, 13, 31):
        v = {mode: _head_mse(wl, 0, h, 128, mode) for mode in O.MODES}
        assert v[O.SYSTEMATIC] <= v[O.STRATIFIED] <= v[O.IID], (h, v)
