"""GPU parity of santa_bernoulli_qk and of the feature-major packing kernel."""

import functools

import numpy as np
import pytest
import torch

from oracle import santa as O
from stochastic_sparse_decode_amd import santa
from stochastic_sparse_decode_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def run_bernoulli(wl, S, mode, seed):
    q, K, V, nk = P.to_dev(wl)
    K_fm = santa.santa_pack_k_feature_major(K)
    B, Hq = wl.B, wl.Hq
    idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hq, wl.max_n_k), float("nan"), dtype=torch.float32, device="cuda")
    kept = torch.full((B, Hq, wl.d), 7, dtype=torch.uint8, device="cuda")
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    out = santa.santa_bernoulli_qk(q, K_fm, V, nk, S, mode, seed, wl.scale, indices=idx, scores=sc, kept=kept,
                                   workspace=ws)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0
    return out.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy(), kept.cpu().numpy().astype(bool)


def test_pack_feature_major_is_exact_relayout():
    wl = W.random_case(2, 4, 2, 128, [256, 192], max_n_k=256, seed=1)
    K = torch.from_numpy(wl.K).cuda()
    got = santa.santa_pack_k_feature_major(K).cpu().numpy()
    assert np.array_equal(got.view(np.uint16), W.feature_major(wl.K).view(np.uint16))
    wl = W.random_case(1, 2, 1, 64, [128], seed=2)
    got = santa.santa_pack_k_feature_major(torch.from_numpy(wl.K).cuda()).cpu().numpy()
    assert np.array_equal(got.view(np.uint16), W.feature_major(wl.K).view(np.uint16))


CASES = [
    ("gqa4", lambda: W.random_case(2, 8, 2, 128, [4096, 2500], max_n_k=4096, seed=11)),
    ("d64_g1", lambda: W.random_case(1, 2, 2, 64, [1000], max_n_k=1024, seed=12)),
    ("g8", lambda: W.random_case(1, 16, 2, 128, [3000], max_n_k=3008, seed=13)),
    ("bernoulli_n8192", lambda: W.bernoulli(B=2, n_k=8192, seed=1004)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", [2, 1, 0])
def test_bernoulli_parity(name, make, mode):
    wl = make()
    S, seed = 128, 21 + mode
    print("[bernoulli] %s mode=%d B=%d Hq=%d Hkv=%d d=%d n_k=%s" % (name, mode, wl.B, wl.Hq, wl.Hkv, wl.d,
                                                                    list(wl.n_k)), flush=True)
    out_g, idx_g, sc_g, kept_g = run_bernoulli(wl, S, mode, seed)
    out_o, idx_o, kept_o, det = O.bernoulli_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale,
                                                   return_detail=True)
    assert np.array_equal(kept_g, kept_o)  # exact fp64 decision on both sides
    flips = set()
    rep = P.compare_indices(idx_g, idx_o, det, P.BAND, flips)
    print("   %s" % rep, flush=True)
    assert rep.bad == 0
    est = P.oracle_estimate_from_indices(wl.V, idx_g, wl.n_k, wl.Hq, S)
    assert np.abs(out_g - est).max() <= P.OUT_TOL
    # scores of the ternary query
    q_t, _, _ = O.bernoulli_queries(wl.q, wl.Hkv, seed)
    s_o = O.all_scores(q_t, wl.K, wl.n_k, wl.scale)
    m = ~np.isnan(s_o)
    assert np.abs(sc_g[m] - s_o[m]).max() <= 1e-4 * max(1.0, np.abs(s_o[m]).max())


def test_bernoulli_equal_magnitudes_match_plain_decode():
    wl = W.random_case(1, 8, 2, 128, [2048], seed=14)
    wl.q[:] = np.where(np.random.default_rng(3).random(wl.q.shape) < 0.5, -0.5, 0.5).astype(np.float16)
    out_b, idx_b, _, kept = run_bernoulli(wl, 64, 2, 4)
    assert kept.all()
    q, K, V, nk = P.to_dev(wl)
    idx = torch.empty((1, 8, 64), dtype=torch.int32, device="cuda")
    santa.santa_decode(q, K, V, nk, 64, 2, 4, wl.scale, indices=idx)
    torch.cuda.synchronize()
    # every feature kept: q~ = q, so both steps sample the oracle's plain
    # decode indices (up to the band at CDF boundaries)
    _, idx_o, det = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, 64, 2, 4, wl.scale, return_detail=True)
    for got in (idx_b, idx.cpu().numpy()):
        rep = P.compare_indices(got, idx_o, det, P.BAND)
        print("   %s" % rep, flush=True)
        assert rep.bad == 0, rep


# the Bernoulli workload at its full size (B=8, n_k=32768, 32/8 heads,
# d=128): full launch, oracle on one sampled head per sequence
@functools.lru_cache(maxsize=1)
def c5_case():
    return W.bernoulli(B=8, n_k=32768, seed=1004)


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_bernoulli_full_size_sampled_heads(mode):
    wl = c5_case()
    S, seed = 128, 51 + mode
    print("[bernoulli] full size B=8 n_k=32768 mode=%d" % mode, flush=True)
    out_g, idx_g, sc_g, kept_g = run_bernoulli(wl, S, mode, seed)
    q_t, kept_o, _ = O.bernoulli_queries(wl.q, wl.Hkv, seed)
    assert np.array_equal(kept_g, kept_o)  # every head: exact decision on both sides
    G = wl.Hq // wl.Hkv
    rep = P.IndexReport()
    for b in range(wl.B):
        h = (7 * b + 3) % wl.Hq
        n = int(wl.n_k[b])
        s = O.head_scores(q_t[b, h], wl.K[b, h // G, :n].astype(np.float64), wl.scale)
        _, _, F = O.distribution(s)
        t = O.points(mode, S, seed, b * wl.Hq + h)
        rep.add(P.compare_head(idx_g[b, h], O.inverse_cdf(F, t), t, F, P.BAND))
        est = O.gather_average(wl.V[b, h // G, :n].astype(np.float64), idx_g[b, h], S)
        assert np.abs(out_g[b, h] - est).max() <= P.OUT_TOL
        assert np.abs(sc_g[b, h, :n] - s).max() <= 1e-4 * max(1.0, np.abs(s).max())
    print("   sampled heads: %s" % rep, flush=True)
    assert rep.bad == 0, rep
    for b in range(wl.B):
        assert np.all(np.diff(idx_g[b], axis=-1) >= 0) and idx_g[b].min() >= 0 and idx_g[b].max() < wl.n_k[b]
    assert np.isfinite(out_g).all()


# more items than resident one-item workgroups: the persistent Bernoulli
# variant, with ragged and invalid lengths (n_k = 0 and n_k > max_n_k)
@functools.lru_cache(maxsize=1)
def persistent_case():
    B, max_n_k = 36, 8192
    rng = np.random.default_rng(77)
    n_k = rng.integers(1, max_n_k + 1, size=B).astype(np.int32)
    n_k[5], n_k[30] = 0, max_n_k + 1
    return W.random_case(B, 32, 8, 128, n_k, max_n_k=max_n_k, seed=78, pad_value=np.float16(np.nan))


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_bernoulli_persistent_parity(mode):
    wl = persistent_case()
    assert wl.B * wl.Hkv * (wl.max_n_k // 1024) > 2048
    S, seed = 64, 31 + mode
    print("[bernoulli] persistent mode=%d B=%d n_k=%s" % (mode, wl.B, list(wl.n_k)[:6]), flush=True)
    out_g, idx_g, sc_g, kept_g = run_bernoulli(wl, S, mode, seed)
    valid = (wl.n_k >= 1) & (wl.n_k <= wl.max_n_k)
    assert np.isnan(out_g[~valid]).all() and (idx_g[~valid] == -1).all()
    out_o, idx_o, kept_o, det = O.bernoulli_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale,
                                                   return_detail=True)
    assert np.array_equal(kept_g[valid], kept_o[valid])
    rep = P.compare_indices(idx_g, idx_o, det, P.BAND)
    print("   %s" % rep, flush=True)
    assert rep.bad == 0
    est = P.oracle_estimate_from_indices(wl.V, idx_g, wl.n_k, wl.Hq, S)
    assert np.abs(out_g[valid] - est[valid]).max() <= P.OUT_TOL
    q_t, _, _ = O.bernoulli_queries(wl.q, wl.Hkv, seed)
    s_o = O.all_scores(q_t, wl.K, wl.n_k, wl.scale)
    m = ~np.isnan(s_o)
    assert np.abs(sc_g[m] - s_o[m]).max() <= 1e-4 * max(1.0, np.abs(s_o[m]).max())


# --------------------------------------------------------------------------
# budget variant: keep probability min(1, m |q| / ||q||_1), value q / pi
# --------------------------------------------------------------------------

def run_budget(wl, S, mode, seed, m):
    q, K, V, nk = P.to_dev(wl)
    K_fm = santa.santa_pack_k_feature_major(K)
    B, Hq = wl.B, wl.Hq
    idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hq, wl.max_n_k), float("nan"), dtype=torch.float32, device="cuda")
    kept = torch.full((B, Hq, wl.d), 7, dtype=torch.uint8, device="cuda")
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    out = santa.santa_bernoulli_qk(q, K_fm, V, nk, S, mode, seed, wl.scale, indices=idx, scores=sc, kept=kept,
                                   workspace=ws, budget=m)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0
    return out.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy(), kept.cpu().numpy().astype(bool)


BUDGET_CASES = [
    ("gqa4_m16", lambda: W.random_case(2, 8, 2, 128, [4096, 2500], max_n_k=4096, seed=61), 16),
    ("gqa4_m64", lambda: W.random_case(1, 8, 2, 128, [3000], max_n_k=3008, seed=62), 64),
    ("d64_g1_m4", lambda: W.random_case(1, 2, 2, 64, [1000], max_n_k=1024, seed=63), 4),
    ("g8_m32", lambda: W.random_case(1, 16, 2, 128, [3000], max_n_k=3008, seed=64), 32),
]


@pytest.mark.parametrize("name,make,m", BUDGET_CASES, ids=[c[0] for c in BUDGET_CASES])
@pytest.mark.parametrize("mode", [2, 1, 0])
def test_bernoulli_budget_parity(name, make, m, mode):
    wl = make()
    S, seed = 128, 41 + mode
    print("[bernoulli-budget] %s m=%d mode=%d" % (name, m, mode), flush=True)
    out_g, idx_g, sc_g, kept_g = run_budget(wl, S, mode, seed, m)
    out_o, idx_o, kept_o, det = O.bernoulli_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale,
                                                   return_detail=True, budget=m)
    assert np.array_equal(kept_g, kept_o)  # exact integer decision on both sides
    rep = P.compare_indices(idx_g, idx_o, det, P.BAND)
    print("   %s" % rep, flush=True)
    assert rep.bad == 0
    est = P.oracle_estimate_from_indices(wl.V, idx_g, wl.n_k, wl.Hq, S)
    assert np.abs(out_g - est).max() <= P.OUT_TOL
    q_t, _, _ = O.bernoulli_queries(wl.q, wl.Hkv, seed, budget=m)
    s_o = O.all_scores(q_t, wl.K, wl.n_k, wl.scale)
    msk = ~np.isnan(s_o)
    assert np.abs(sc_g[msk] - s_o[msk]).max() <= 1e-4 * max(1.0, np.abs(s_o[msk]).max())
