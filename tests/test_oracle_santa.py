"""Pins for the oracle's score, distribution, sampling and estimate steps (CPU).

Each test checks the oracle against something other than itself: a library
routine (PyTorch's scaled-dot-product attention in fp64), closed forms,
structural properties that the sampling schemes guarantee, or an independent
brute-force search.
"""

import numpy as np
import pytest
import torch

from oracle import philox
from oracle import santa as O
from stochastic_sparse_decode_amd import workloads as W


def _sdpa_reference(wl):
    """Exact attention via torch SDPA (fp64, CPU), KV heads repeated for GQA."""
    B, Hq, Hkv = wl.B, wl.Hq, wl.Hkv
    G = Hq // Hkv
    out = np.zeros((B, Hq, wl.d))
    for b in range(B):
        n = int(wl.n_k[b])
        q = torch.from_numpy(wl.q[b].astype(np.float64))[:, None, :]  # (Hq, 1, d)
        k = torch.from_numpy(wl.K[b, :, :n].astype(np.float64)).repeat_interleave(G, dim=0)
        v = torch.from_numpy(wl.V[b, :, :n].astype(np.float64)).repeat_interleave(G, dim=0)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=wl.scale)
        out[b] = o[:, 0, :].numpy()
    return out


@pytest.mark.parametrize("shape", [(2, 4, 2, 16, [37, 50]), (1, 8, 1, 32, [129]), (3, 6, 3, 8, [1, 5, 64])])
def test_dense_matches_sdpa(shape):
    B, Hq, Hkv, d, n_k = shape
    wl = W.random_case(B, Hq, Hkv, d, n_k, seed=11, q_scale=2.0)
    ref = _sdpa_reference(wl)
    got = O.dense_decode(wl.q, wl.K, wl.V, wl.n_k, wl.scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_dense_planted_llama_shape_matches_sdpa():
    wl = W.llama(B=1, n_k=2048, seed=3)
    ref = _sdpa_reference(wl)
    got = O.dense_decode(wl.q, wl.K, wl.V, wl.n_k, wl.scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_scores_match_float64_matmul_and_gqa_mapping():
    wl = W.random_case(2, 8, 2, 16, [10, 12], seed=4)
    s = O.all_scores(wl.q, wl.K, wl.n_k, wl.scale)
    for b in range(2):
        n = int(wl.n_k[b])
        for h in range(8):
            ref = torch.from_numpy(wl.K[b, h // 4, :n].astype(np.float64)) @ torch.from_numpy(
                wl.q[b, h].astype(np.float64))
            np.testing.assert_allclose(s[b, h, :n], wl.scale * ref.numpy(), rtol=1e-15, atol=1e-15)


def test_uniform_scores_give_mean_of_values():
    """q = 0: every key has weight 1/n, dense output = mean(V)."""
    wl = W.random_case(1, 2, 1, 8, [300], seed=5)
    wl.q[:] = 0
    dense = O.dense_decode(wl.q, wl.K, wl.V, wl.n_k, wl.scale)
    mean = wl.V[0, 0].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(dense[0, 0], mean, rtol=0, atol=1e-14)


@pytest.mark.parametrize("n", [1, 7, 64, 1000])
def test_systematic_with_S_equal_n_and_uniform_p_returns_mean_exactly(n):
    """S = n_k, uniform p: t_k = (k + u)/n lies in [F_{k-1}, F_k), so i_k = k."""
    wl = W.random_case(1, 1, 1, 8, [n], seed=6)
    wl.q[:] = 0
    for seed in range(5):
        out, idx = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, n, O.SYSTEMATIC, seed, wl.scale)
        assert np.array_equal(idx[0, 0], np.arange(n))
        np.testing.assert_allclose(out[0, 0], wl.V[0, 0].astype(np.float64).mean(axis=0),
                                   rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", O.MODES)
def test_one_hot_scores_select_one_key(mode):
    """One logit 120 above the rest: every point lands on that key, o^ = V_j*."""
    d, n, jstar = 4, 50, 17
    q = np.zeros((1, 1, d), dtype=np.float16)
    q[0, 0, 0] = 8.0
    K = np.zeros((1, 1, n, d), dtype=np.float16)
    K[0, 0, jstar, 0] = 15.0  # score 120 at scale 1
    V = np.random.default_rng(0).standard_normal((1, 1, n, d)).astype(np.float16)
    out, idx = O.santa_decode(q, K, V, [n], 32, mode, 123, 1.0)
    assert np.all(idx == jstar)
    np.testing.assert_array_equal(out[0, 0], V[0, 0, jstar].astype(np.float64))


def _walk_search(cum, t):
    """Independent inverse CDF: walk keys until the running sum exceeds t * Z."""
    Z = cum[-1]
    res = []
    for tk in t:
        j = 0
        while j < len(cum) - 1 and cum[j] / Z <= tk:
            j += 1
        res.append(j)
    return np.array(res)


def test_inverse_cdf_matches_linear_walk_including_exact_ties():
    rng = np.random.default_rng(8)
    for trial in range(30):
        n = int(rng.integers(1, 40))
        w = rng.integers(0, 4, size=n).astype(np.float64)  # zero weights included
        if w.sum() == 0:
            w[-1] = 1
        cum = np.cumsum(w)
        F = cum / cum[-1]
        # points on every CDF value (ties), at 0, and random points
        t = np.concatenate((F[:-1], [0.0], rng.random(20)))
        t = np.sort(t[t < 1.0])
        np.testing.assert_array_equal(O.inverse_cdf(F, t), _walk_search(cum, t))


def test_zero_weight_keys_are_never_selected():
    s = np.array([0.0, -np.inf, 0.0, -np.inf, -np.inf, 1.0])
    _, _, F = O.distribution(s)
    for seed in range(50):
        for mode in O.MODES:
            idx = O.inverse_cdf(F, O.points(mode, 16, seed, 0))
            assert not np.isin(idx, [1, 3, 4]).any()


def test_points_follow_the_scheme_definitions():
    S = 64
    for seed in range(20):
        u_sys = philox.uniforms(seed, 3, philox.TAG_SYSTEMATIC, 1)[0]
        t = O.points(O.SYSTEMATIC, S, seed, 3)
        np.testing.assert_array_equal(t, (np.arange(S) + u_sys) / S)
        assert np.all(np.diff(t) == 1.0 / S)  # exact for power-of-two S
        t = O.points(O.STRATIFIED, S, seed, 3)
        k = np.arange(S)
        assert np.all((t >= k / S) & (t < (k + 1) / S))  # one point per stratum
        t = O.points(O.IID, S, seed, 3)
        assert np.all(np.diff(t) >= 0) and t[0] >= 0 and t[-1] < 1
        np.testing.assert_array_equal(np.sort(philox.uniforms(seed, 3, philox.TAG_IID, S)), t)


def _counts(idx, n):
    return np.bincount(idx, minlength=n)


def test_systematic_counts_are_floor_or_ceil_of_S_p():
    rng = np.random.default_rng(9)
    for trial in range(40):
        n = int(rng.integers(2, 200))
        S = int(rng.choice([3, 16, 50, 128]))
        s = 3.0 * rng.standard_normal(n)
        p = O.probabilities(s)
        _, _, F = O.distribution(s)
        idx = O.inverse_cdf(F, O.points(O.SYSTEMATIC, S, trial, 0))
        c = _counts(idx, n)
        assert c.sum() == S
        assert np.all(c >= np.floor(S * p - 1e-9)) and np.all(c <= np.ceil(S * p + 1e-9))


def test_stratified_counts_within_one_of_S_p():
    rng = np.random.default_rng(10)
    for trial in range(40):
        n = int(rng.integers(2, 200))
        S = int(rng.choice([3, 16, 50, 128]))
        s = 3.0 * rng.standard_normal(n)
        p = O.probabilities(s)
        _, _, F = O.distribution(s)
        idx = O.inverse_cdf(F, O.points(O.STRATIFIED, S, trial, 0))
        assert np.all(np.diff(idx) >= 0)
        c = _counts(idx, n)
        assert np.all(c >= np.floor(S * p - 1e-9) - 1) and np.all(c <= np.ceil(S * p + 1e-9) + 1)


def test_iid_counts_chi_square_against_p():
    """Pooled i.i.d. counts over 10^4 seeds follow the multinomial law p."""
    rng = np.random.default_rng(12)
    n, S, seeds = 12, 16, 10000
    s = rng.standard_normal(n)
    p = O.probabilities(s)
    _, _, F = O.distribution(s)
    pooled = np.zeros(n)
    for seed in range(seeds):
        pooled += _counts(O.inverse_cdf(F, O.points(O.IID, S, seed, 0)), n)
    expected = p * S * seeds
    chi2 = ((pooled - expected) ** 2 / expected).sum()
    assert chi2 < 40.0  # 11 dof; p ~ 4e-5


def test_gather_average_counts_duplicates():
    V = np.arange(12, dtype=np.float64).reshape(4, 3)
    got = O.gather_average(V, [1, 1, 3, 0], 4)
    np.testing.assert_array_equal(got, (2 * V[1] + V[3] + V[0]) / 4)


def test_invalid_sequence_length_yields_nan_and_minus_one():
    wl = W.random_case(2, 2, 1, 8, [5, 5], seed=13)
    n_k = np.array([0, 6])  # 0 and > max_n_k are both invalid
    out, idx = O.santa_decode(wl.q, wl.K, wl.V, n_k, 4, O.SYSTEMATIC, 1, wl.scale)
    assert np.isnan(out).all() and (idx == -1).all()
    assert np.isnan(O.dense_decode(wl.q, wl.K, wl.V, n_k, wl.scale)).all()


def test_score_override_reproduces_normal_path():
    wl = W.random_case(2, 4, 2, 16, [40, 33], seed=14)
    s = O.all_scores(wl.q, wl.K, wl.n_k, wl.scale)
    a = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, 8, O.STRATIFIED, 5, wl.scale)
    b = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, 8, O.STRATIFIED, 5, wl.scale, score_override=s)
    np.testing.assert_array_equal(a[1], b[1])
    np.testing.assert_array_equal(a[0], b[0])


# --------------------------------------------------------------------------
# Bernoulli qK^T
# --------------------------------------------------------------------------

def test_ternary_query_is_unbiased():
    """E[q~] = q: mean over 10^4 draws within 4 sigma for every feature."""
    rng = np.random.default_rng(15)
    qg = rng.standard_normal((4, 32))
    N = 10000
    acc = np.zeros_like(qg)
    for seed in range(N):
        u = philox.uniforms(seed, 0, philox.TAG_BERNOULLI, 32)
        qt, kept, A = O.ternary_query(qg, u)
        acc += qt
    A = np.abs(qg).max(axis=1, keepdims=True)
    var = A * np.abs(qg) - qg ** 2  # Var of sign(q) A Bernoulli(|q|/A)
    z = (acc / N - qg) / np.sqrt(np.maximum(var, 1e-300) / N)
    z[var == 0] = 0
    assert np.abs(z).max() < 4.5


def test_ternary_query_structure():
    rng = np.random.default_rng(16)
    qg = rng.standard_normal((2, 64)).astype(np.float16).astype(np.float64)
    u = philox.uniforms(4, 0, philox.TAG_BERNOULLI, 64)
    qt, kept, A = O.ternary_query(qg, u)
    # exactly ternary {-A, 0, +A}; the largest |q| is always kept
    for h in range(2):
        assert set(np.unique(np.abs(qt[h]))) <= {0.0, A[h]}
        assert kept[h, np.argmax(np.abs(qg[h]))]
    assert np.array_equal(np.sign(qt[kept]), np.sign(qg[kept]))


def test_bernoulli_equal_magnitudes_keep_everything():
    """All |q_i| equal: keep probability 1, so q~ = q and scores are exact."""
    wl = W.random_case(1, 4, 2, 16, [40], seed=17)
    wl.q[:] = np.where(np.random.default_rng(1).random(wl.q.shape) < 0.5, -0.75, 0.75)
    out_b, idx_b, kept = O.bernoulli_decode(wl.q, wl.K, wl.V, wl.n_k, 8, O.SYSTEMATIC, 3, wl.scale)
    out_s, idx_s = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, 8, O.SYSTEMATIC, 3, wl.scale)
    assert kept.all()
    np.testing.assert_array_equal(idx_b, idx_s)
    np.testing.assert_array_equal(out_b, out_s)


def test_bernoulli_zero_query_gives_uniform_distribution():
    wl = W.random_case(1, 1, 1, 8, [64], seed=18)
    wl.q[:] = 0
    out, idx, kept = O.bernoulli_decode(wl.q, wl.K, wl.V, wl.n_k, 64, O.SYSTEMATIC, 2, wl.scale)
    assert not kept.any()
    assert np.array_equal(idx[0, 0], np.arange(64))


def test_bernoulli_kept_count_expectation():
    rng = np.random.default_rng(19)
    qg = rng.standard_normal((1, 128))
    pi = np.abs(qg[0]) / np.abs(qg[0]).max()
    counts = [O.ternary_query(qg, philox.uniforms(s, 0, philox.TAG_BERNOULLI, 128))[1].sum()
              for s in range(4000)]
    sd = np.sqrt((pi * (1 - pi)).sum() / len(counts))
    assert abs(np.mean(counts) - pi.sum()) < 4 * sd


def _bern_uniforms_from_core(seed, row, d):
    """Uniform i of stream (seed, row, 'BERN') computed from the Philox core
    itself (pinned by the generator authors' vectors): word i & 3 of the block
    at counter (i >> 2, row, tag, 0), key (seed lo, seed hi), as (x >> 8) 2^-24."""
    u = np.zeros(d)
    for i in range(d):
        words = philox.philox4x32_10(i >> 2, row, philox.TAG_BERNOULLI, 0, seed & 0xFFFFFFFF, seed >> 32)
        u[i] = float(int(words[i & 3]) >> 8) * 2.0 ** -24
    return u


def test_bernoulli_queries_stream_rows_and_group_sharing():
    """One draw of d uniforms per KV head (b, h_kv), from stream row
    b * H_kv + h_kv, shared by the group's G query heads (a draw per query
    head, or the row b * H_q + h, fails here)."""
    B, Hkv, G, d = 3, 2, 4, 64
    Hq = Hkv * G
    rng = np.random.default_rng(23)
    mag = np.abs(rng.standard_normal(d)).astype(np.float16)
    signs = rng.choice([-1.0, 1.0], size=(B, Hq, d))
    q = (mag[None, None, :] * signs).astype(np.float16)  # every head has the same |q|
    seed = (7 << 32) | 99
    _, kept, A = O.bernoulli_queries(q, Hkv, seed)
    qa = np.abs(q.astype(np.float64))
    wrong_row_differs = False
    for b in range(B):
        for hk in range(Hkv):
            heads = range(hk * G, (hk + 1) * G)
            u = _bern_uniforms_from_core(seed, b * Hkv + hk, d)
            for h in heads:
                # equal |q| in the group: one shared mask, the rule u A < |q| on this row
                assert np.array_equal(kept[b, h], u * A[b, h] < qa[b, h])
                assert np.array_equal(kept[b, h], kept[b, hk * G])
            u_wrong = _bern_uniforms_from_core(seed, b * Hq + hk * G + 1, d)
            wrong_row_differs |= not np.array_equal(kept[b, hk * G], u_wrong * A[b, hk * G] < qa[b, hk * G])
    assert wrong_row_differs
    # the same |q| in the other groups and sequences: each draws its own mask
    masks = {kept[b, hk * G].tobytes() for b in range(B) for hk in range(Hkv)}
    assert len(masks) == B * Hkv


# --------------------------------------------------------------------------
# Bernoulli budget variant: pi = min(1, m |q| / ||q||_1), kept value q / pi
# --------------------------------------------------------------------------

def test_budget_query_is_unbiased():
    """E[q~] = q: mean over 10^4 draws within 4.5 sigma for every feature."""
    rng = np.random.default_rng(21)
    qg = rng.standard_normal((2, 32)).astype(np.float16).astype(np.float64)
    m = 8
    N = 10000
    acc = np.zeros_like(qg)
    for seed in range(N):
        u = philox.uniforms(seed, 0, philox.TAG_BERNOULLI, 32)
        acc += O.budget_query(qg, u, m)[0]
    L1 = np.abs(qg).sum(axis=1, keepdims=True)
    pi = np.minimum(1.0, m * np.abs(qg) / L1)
    var = qg ** 2 * (1.0 / pi - 1.0)  # Var of (q / pi) Bernoulli(pi)
    z = (acc / N - qg) / np.sqrt(np.maximum(var, 1e-300) / N)
    z[var == 0] = 0
    assert np.abs(z).max() < 4.5


def test_budget_query_structure_and_exact_decision():
    rng = np.random.default_rng(22)
    qg = (rng.standard_normal((3, 64)) * np.array([[1.0], [0.01], [30.0]])).astype(np.float16).astype(np.float64)
    u = philox.uniforms(5, 0, philox.TAG_BERNOULLI, 64)
    for m in (1, 4, 16, 64):
        qt, kept, clipped, c = O.budget_query(qg, u, m)
        L1 = np.abs(qg).sum(axis=1)
        assert np.allclose(c, L1 / m, rtol=1e-15)
        pi = np.minimum(1.0, m * np.abs(qg) / L1[:, None])
        # clipped exactly where pi = 1; clipped features are always kept, at q
        assert np.array_equal(clipped, m * np.abs(qg) >= L1[:, None])
        assert kept[clipped].all() and np.array_equal(qt[clipped], qg[clipped])
        # unclipped kept features take sign(q) ||q||_1 / m
        uk = kept & ~clipped
        assert np.allclose(np.abs(qt[uk]), np.broadcast_to(c[:, None], qt.shape)[uk], rtol=1e-15)
        assert np.array_equal(np.sign(qt[kept]), np.sign(qg[kept]))
        # the decision agrees with the fp64 comparison u < pi wherever that
        # comparison is not within rounding of a tie
        margin = np.abs(u[None, :] - pi) > 1e-12
        assert np.array_equal(kept[margin], (u[None, :] < pi)[margin])


def test_budget_query_clips_everything_when_the_budget_covers_all():
    qg = np.full((2, 16), 0.5)
    qg[1, ::2] = -0.25
    qg[1, 1::2] = 0.25
    u = philox.uniforms(3, 0, philox.TAG_BERNOULLI, 16)
    qt, kept, clipped, _ = O.budget_query(qg, u, 16)   # m |q_i| >= ||q||_1 for equal magnitudes
    assert clipped.all() and kept.all() and np.array_equal(qt, qg)
    qt, kept, _, _ = O.budget_query(np.zeros((1, 16)), u, 4)
    assert not kept.any() and not qt.any()


def test_budget_kept_count_expectation():
    rng = np.random.default_rng(23)
    qg = rng.standard_normal((1, 128)).astype(np.float16).astype(np.float64)
    m = 24
    pi = np.minimum(1.0, m * np.abs(qg[0]) / np.abs(qg[0]).sum())
    counts = [O.budget_query(qg, philox.uniforms(s, 0, philox.TAG_BERNOULLI, 128), m)[1].sum()
              for s in range(2000)]
    sd = np.sqrt((pi * (1 - pi)).sum() / len(counts))
    assert abs(np.mean(counts) - pi.sum()) < 4 * sd
    assert pi.sum() <= m + 1e-9
