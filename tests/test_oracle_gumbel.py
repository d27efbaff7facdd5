"""Pins for the oracle's Gumbel-max i.i.d. sampler (mode 3), CPU only.

The sampler's stream is checked against the Philox core itself (pinned by the
generator authors' vectors), its outcomes against closed cases (a dominant
logit; equal logits, where the draw is the largest raw uniform), and its law
against the softmax: a chi-square test of pooled counts and the mean estimate
over many seeds within 3 sigma of dense attention (sigma from the exact
i.i.d. variance)."""

import numpy as np
from scipy import stats

from oracle import moments as M
from oracle import philox
from oracle import santa as O
from stochastic_sparse_decode_amd import workloads as W


def test_draw_uniforms_follow_the_counter_layout():
    seed, row = (5 << 32) | 77, 9
    for draw in (0, 3, 1000):
        u = philox.draw_uniforms(seed, row, philox.TAG_GUMBEL, draw, 11)
        for j in range(11):
            words = philox.philox4x32_10(j >> 2, row, philox.TAG_GUMBEL, draw, seed & 0xFFFFFFFF, seed >> 32)
            assert u[j] == ((int(words[j & 3]) >> 9) + 0.5) * 2.0 ** -23
        assert np.all((u > 0) & (u < 1))
    # the draw index moves the counter: different draws, different words
    a = philox.draw_uniforms(seed, row, philox.TAG_GUMBEL, 0, 8)
    b = philox.draw_uniforms(seed, row, philox.TAG_GUMBEL, 1, 8)
    assert not np.array_equal(a, b)


def test_dominant_logit_wins_every_draw():
    # the Gumbel transform of the open-interval 23-bit uniforms lies in
    # [-2.82, 16.7], so a logit 40 above the others wins every draw
    s = np.zeros(50)
    s[17] = 40.0
    idx, gap = O.gumbel_draws(s, 64, 3, 0)
    assert np.all(idx == 17) and np.all(gap > 20)


def test_equal_logits_take_the_largest_uniform():
    s = np.full(37, -1.25)
    seed, row = 11, 4
    idx, _ = O.gumbel_draws(s, 20, seed, row)
    for k in range(20):
        u = philox.draw_uniforms(seed, row, philox.TAG_GUMBEL, k, 37)
        assert idx[k] == int(np.argmax(u))  # -log(-log u) increases with u


def test_counts_follow_the_softmax():
    rng = np.random.default_rng(3)
    s = rng.standard_normal(12)
    p = np.exp(s - s.max())
    p /= p.sum()
    counts = np.zeros(12)
    for seed in range(150):
        idx, _ = O.gumbel_draws(s, 200, seed, 0)
        counts += np.bincount(idx, minlength=12)
    chi2, pval = stats.chisquare(counts, counts.sum() * p)
    assert pval > 1e-3, (chi2, pval)


def test_mean_over_seeds_matches_dense_attention():
    wl = W.random_case(1, 1, 1, 16, [48], seed=21, planted=True)
    s = O.head_scores(wl.q[0, 0].astype(np.float64), wl.K[0, 0].astype(np.float64), wl.scale)
    _, _, F = O.distribution(s)
    Vh = wl.V[0, 0].astype(np.float64)
    dense = O.dense_head(s, Vh)
    N, S = 2000, 8
    est = np.zeros((N, wl.d))
    for seed in range(N):
        idx, _ = O.gumbel_draws(s, S, seed, 0)
        est[seed] = O.gather_average(Vh, idx, S)
    _, var = M.moments(O.IID, F, Vh, S)  # the law of i.i.d. draws
    z = (est.mean(axis=0) - dense) / np.sqrt(var / N)
    assert np.abs(z).max() < 4.5 and (np.abs(z) > 3).sum() <= 1, z


def test_decode_mode_3_sorts_the_draws_and_averages():
    wl = W.random_case(1, 4, 2, 16, [60], seed=22)
    out, idx, det = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, 16, O.GUMBEL, 5, wl.scale, return_detail=True)
    for h in range(4):
        assert np.all(np.diff(idx[0, h]) >= 0)
        assert np.all(det["gap"][(0, h)] > 0)
    s = O.head_scores(wl.q[0, 1].astype(np.float64), wl.K[0, 0, :60].astype(np.float64), wl.scale)
    raw, _ = O.gumbel_draws(s, 16, 5, 1)
    assert np.array_equal(np.sort(raw), idx[0, 1])
