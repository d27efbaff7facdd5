"""GPU parity of santa_decode against the fp64 oracle (through the C-ABI).

Index parity: bit-exact except for points within 1e-5 of every CDF value that
separates the GPU's and the oracle's choice (counted and printed); a second
check re-runs the oracle's sampling steps on the GPU's own fp32 scores, where
the excused band shrinks to 1e-6.  Output parity: max-abs 2e-3 against the
oracle's estimate on the GPU's index list, and against the oracle's own output
for every head without a flip.
"""

import functools

import numpy as np
import pytest
import torch

from oracle import santa as O
from stochastic_sparse_decode_amd import santa
from stochastic_sparse_decode_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def run_decode(wl, S, mode, seed, workspace=None, with_scores=True):
    q, K, V, nk = P.to_dev(wl)
    B, Hq = wl.B, wl.Hq
    idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hq, wl.max_n_k), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    ws = workspace if workspace is not None else santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    out = santa.santa_decode(q, K, V, nk, S, mode, seed, wl.scale, indices=idx, scores=sc, workspace=ws)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0
    return out.cpu().numpy(), idx.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def check_parity(wl, S, mode, seed, label=""):
    print("[decode] %s S=%d mode=%d seed=%d B=%d Hq=%d Hkv=%d d=%d n_k=%s" % (
        label, S, mode, seed, wl.B, wl.Hq, wl.Hkv, wl.d, list(wl.n_k)[:4]), flush=True)
    out_g, idx_g, sc_g = run_decode(wl, S, mode, seed)
    out_o, idx_o, det = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale, return_detail=True)
    valid = (wl.n_k >= 1) & (wl.n_k <= wl.max_n_k)
    # index lists are ascending and inside [0, n_k)
    for b in np.nonzero(valid)[0]:
        assert np.all(np.diff(idx_g[b], axis=-1) >= 0)
        assert idx_g[b].min() >= 0 and idx_g[b].max() < wl.n_k[b]
    flips = set()
    rep = P.compare_indices(idx_g, idx_o, det, P.BAND, flips)
    _, idx_s, det_s = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale,
                                     score_override=sc_g, return_detail=True)
    rep2 = P.compare_indices(idx_g, idx_s, det_s, P.BAND_SAME_SCORES)
    print("   vs oracle: %s | on GPU scores: %s" % (rep, rep2), flush=True)
    assert rep.bad == 0, rep
    assert rep2.bad == 0, rep2
    est = P.oracle_estimate_from_indices(wl.V, idx_g, wl.n_k, wl.Hq, S)
    err = np.abs(out_g[valid] - est[valid]).max()
    assert err <= P.OUT_TOL, err
    for b in np.nonzero(valid)[0]:
        for h in range(wl.Hq):
            if (b, h) not in flips:
                assert np.abs(out_g[b, h] - out_o[b, h]).max() <= P.OUT_TOL
    # score stage against the oracle's fp64 scores
    s_o = O.all_scores(wl.q, wl.K, wl.n_k, wl.scale)
    m = ~np.isnan(s_o)
    assert np.abs(sc_g[m] - s_o[m]).max() <= 1e-4 * max(1.0, np.abs(s_o[m]).max())
    return rep


# --------------------------------------------------------------------------
# tiny single-head config (d=64, n_k=1024, 4 planted keys, scale folded in q)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [2, 1, 0])
@pytest.mark.parametrize("S", [16, 1, 1000])
def test_tiny_parity(mode, S):
    wl = W.tiny()
    for seed in range(3):
        check_parity(wl, S, mode, seed, "tiny")


def test_tiny_systematic_S_equals_n_uniform_is_mean_exactly():
    wl = W.tiny()
    wl.q[:] = 0
    out, idx, _ = run_decode(wl, 1024, 2, 7)
    assert np.array_equal(idx[0, 0], np.arange(1024))
    ref = wl.V[0, 0].astype(np.float64).mean(axis=0)
    assert np.abs(out[0, 0] - ref).max() < 1e-6


# --------------------------------------------------------------------------
# GQA packing, head dims, ragged tails, padding poisoned with NaN
# --------------------------------------------------------------------------

SMALL = [
    # B, Hq, Hkv, d, n_k, max_n_k
    (2, 8, 2, 128, [3000, 1500], 3100),
    (1, 4, 4, 128, [2049], 2049),
    (2, 4, 2, 64, [1024, 1], 1024),
    (1, 16, 2, 128, [4500], 4500),
    (3, 8, 4, 64, [777, 2048, 1025], 2100),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d" % c[:4])
@pytest.mark.parametrize("mode", [2, 1, 0])
def test_small_shapes_parity(case, mode):
    B, Hq, Hkv, d, n_k, max_n_k = case
    wl = W.random_case(B, Hq, Hkv, d, n_k, max_n_k=max_n_k, seed=31 + B + d, planted=True,
                       pad_value=np.float16(np.nan))
    for S in (8, 128):
        check_parity(wl, S, mode, 100 + S, "small")


def test_invalid_sequence_lengths():
    wl = W.random_case(3, 8, 2, 128, [0, 1200, 5000], max_n_k=2048, seed=5)
    out, idx, _ = run_decode(wl, 16, 2, 3)
    assert np.isnan(out[0]).all() and (idx[0] == -1).all()
    assert np.isnan(out[2]).all() and (idx[2] == -1).all()
    assert not np.isnan(out[1]).any()
    check_parity(wl, 16, 2, 3, "invalid-n_k")


# --------------------------------------------------------------------------
# more items than one workgroup per CU: the persistent, pipelined variant
# (workgroups take the valid splits round-robin); ragged and invalid lengths,
# and more than 64 sequences (several chunks of the per-sequence item count)
# --------------------------------------------------------------------------

PERSISTENT = [
    # B, Hq, Hkv, d, max_n_k, invalid sequences (n_k set to 0 or max_n_k + 1);
    # over 2048 items, more than any number of resident one-item workgroups
    (20, 32, 8, 128, 16384, (3, 11)),
    (70, 1, 1, 64, 32768, (0, 65, 69)),
]


@functools.lru_cache(maxsize=2)
def persistent_case(case):
    B, Hq, Hkv, d, max_n_k, bad = case
    rng = np.random.default_rng(B + d)
    n_k = rng.integers(1, max_n_k + 1, size=B).astype(np.int32)
    for i, bi in enumerate(bad):
        n_k[bi] = 0 if i % 2 == 0 else max_n_k + 1
    return W.random_case(B, Hq, Hkv, d, n_k, max_n_k=max_n_k, seed=B + 7, planted=True,
                         pad_value=np.float16(np.nan))


@pytest.mark.parametrize("case", PERSISTENT, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d" % c[:4])
@pytest.mark.parametrize("mode", [2, 1, 0])
def test_persistent_ragged_invalid_parity(case, mode):
    wl = persistent_case(case)
    assert wl.B * wl.Hkv * ((wl.max_n_k + 1023) // 1024) > 2048
    out, idx, _ = run_decode(wl, 32, mode, 17, with_scores=False)
    for bi in case[5]:
        assert np.isnan(out[bi]).all() and (idx[bi] == -1).all()
    check_parity(wl, 32, mode, 17, "persistent")


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_group_beyond_register_chunks_parity(mode):
    # one KV head with 294 splits: more than the 256 whose slots are read into
    # registers at once, so the waits and the merge also take the chunk-wise
    # path (the pipelined variant: 294 items exceed one per CU)
    wl = W.random_case(1, 4, 1, 64, [300123], max_n_k=300123, seed=77, planted=True)
    assert (wl.max_n_k + 1023) // 1024 > 256
    check_parity(wl, 128, mode, 23, "long group")


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_short_splits_beyond_register_chunks_parity(mode):
    # one KV head with 391 splits of 512 keys (200000 keys: fewer than two
    # 1024-key splits per CU, so the 512-key variant runs): more than the 256
    # splits whose slots are read into registers at once
    wl = W.random_case(1, 4, 1, 64, [200000], max_n_k=200000, seed=79, planted=True)
    check_parity(wl, 128, mode, 25, "long group, short splits")
    out_g, idx_g = run_decode_det(wl, 128, mode, 25)
    _one_rounding(out_g, idx_g, wl, 128)


# --------------------------------------------------------------------------
# Llama-3.1-8B decode layer at 32k (32 q heads, 8 KV heads, d=128)
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def llama32k():
    return W.llama(B=1, n_k=32768, seed=1001)


@pytest.mark.parametrize("mode", [2, 1, 0])
@pytest.mark.parametrize("S", [32, 64, 128, 256])
def test_llama32k_parity(llama32k, mode, S):
    check_parity(llama32k, S, mode, 1 + S, "llama32k")


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_llama32k_max_S(llama32k, mode):
    # many points per split: most lanes of the heavy splits hold points
    check_parity(llama32k, 1024, mode, 9, "llama32k")


def test_llama32k_bench_call_index_free(llama32k):
    """The call the benchmark times: systematic, S=128, seed 1, no indices, no
    scores.  Its output is compared with the oracle's output for every head
    whose points all lie farther than the band from every CDF value (those
    heads' indices are determined); the other heads are counted, and for them
    the output must match the oracle's estimate on the index list that the
    same call returns when asked for indices."""
    wl = llama32k
    S, mode, seed = 128, 2, 1
    q, K, V, nk = P.to_dev(wl)
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    out = santa.santa_decode(q, K, V, nk, S, mode, seed, wl.scale, workspace=ws)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0
    out = out.cpu().numpy()
    out_o, idx_o, det = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale, return_detail=True)
    clean, near = 0, []
    for h in range(wl.Hq):
        if P.min_boundary_distance(det["t"][(0, h)], det["F"][(0, h)]) > P.BAND:
            clean += 1
            err = np.abs(out[0, h] - out_o[0, h]).max()
            assert err <= P.OUT_TOL, (h, err)
        else:
            near.append(h)
    print("   index-free bench call: %d heads compared with the oracle, %d heads with a point within %g of a "
          "CDF value" % (clean, len(near), P.BAND), flush=True)
    # the same call with indices: identical output, and indices that pass the band rule
    idx = torch.empty((1, wl.Hq, S), dtype=torch.int32, device="cuda")
    out2 = santa.santa_decode(q, K, V, nk, S, mode, seed, wl.scale, indices=idx, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out2.cpu().numpy(), out, rtol=0, atol=1e-6)
    idx = idx.cpu().numpy()
    rep = P.compare_indices(idx, idx_o, det, P.BAND)
    print("   indices: %s" % rep, flush=True)
    assert rep.bad == 0
    est = P.oracle_estimate_from_indices(wl.V, idx, wl.n_k, wl.Hq, S)
    assert np.abs(out - est).max() <= P.OUT_TOL


def test_workspace_shared_by_sampling_and_dense_problems():
    """One workspace serves sampling and dense steps of different sizes in
    turn: a B=1 sampling step, then a B=16 dense step, and a dense step with
    33 splits per KV head whose arrival counters land on the sampling step's
    statistics slots (tagged values, not zeros).  The dense results match the
    oracle every time."""
    small = W.llama(B=1, n_k=32768, seed=5)
    big = W.llama(B=16, n_k_range=(1500, 3000), max_n_k=32768, seed=4, pad_value=np.float16(np.nan))
    over = W.llama(B=1, n_k=33000, max_n_k=33792, seed=6, pad_value=np.float16(np.nan))
    qs, Ks, Vs, nks = P.to_dev(small)
    dense_cases = []
    for wl in (big, over):
        qd, Kd, Vd, nkd = P.to_dev(wl)
        dense_cases.append((wl, (qd, Kd, Vd, nkd), O.dense_decode(wl.q, wl.K, wl.V, wl.n_k, wl.scale)))
    need = max(santa.workspace_bytes(santa.problem(t[0], t[1], wl.scale)) for wl, t, _ in dense_cases)
    need = max(need, santa.workspace_bytes(santa.problem(qs, Ks, small.scale)))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for wl, (qd, Kd, Vd, nkd), ref in dense_cases:
            santa.santa_decode(qs, Ks, Vs, nks, 128, 2, 3 + rep, small.scale, workspace=ws)
            got = santa.santa_dense_decode(qd, Kd, Vd, nkd, wl.scale, workspace=ws)
            torch.cuda.synchronize()
            assert santa.santa_workspace_error(ws) == 0
            err = np.abs(got.cpu().numpy() - ref).max()
            print("   rep %d B=%d max_n_k=%d: dense max abs err %.3g" % (rep, wl.B, wl.max_n_k, err), flush=True)
            assert err <= P.DENSE_TOL


def run_decode_det(wl, S, mode, seed, workspace=None):
    q, K, V, nk = P.to_dev(wl)
    idx = torch.full((wl.B, wl.Hq, S), -7, dtype=torch.int32, device="cuda")
    ws = workspace if workspace is not None else santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    out = santa.santa_decode(q, K, V, nk, S, mode, seed, wl.scale, indices=idx, workspace=ws, deterministic=True)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0
    return out.cpu().numpy(), idx.cpu().numpy()


def _same(x, y):
    """Deterministic mode: indices and outputs bit-identical."""
    assert np.array_equal(x[1], y[1])
    assert np.array_equal(x[0].view(np.uint32), y[0].view(np.uint32))


def test_determinism_and_workspace_reuse(llama32k):
    """Bit-identical results over repeated runs (SANTA_DETERMINISTIC); one
    workspace shared by a large and a small problem."""
    wl = llama32k
    q, K, V, nk = P.to_dev(wl)
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    small = W.random_case(2, 8, 2, 128, [3000, 1500], max_n_k=3100, seed=2)
    small_fresh = run_decode_det(small, 64, 1, 5)
    a = run_decode_det(wl, 128, 2, 11, workspace=ws)
    for _ in range(3):
        sm = run_decode_det(small, 64, 1, 5, workspace=ws)
        b = run_decode_det(wl, 128, 2, 11, workspace=ws)
        _same(a, b)
        _same(sm, small_fresh)
    assert santa.santa_workspace_error(ws) == 0


def test_launch_tags_across_variants_and_grids(llama32k):
    """One workspace serves, in turn, launches of every sampling variant with
    different grids: one workgroup per CU (the Llama layer), two per CU with
    512-key splits (B = 4 at 4096 keys; B = 2, 3100 keys), and the persistent
    variant (B = 6, up to 20480 keys).  Each launch derives its tag from the
    workspace's launch counters and must accept no statistics slot of an
    earlier launch: every repeat reproduces its problem's first result bit for
    bit (deterministic mode)."""
    wls = [llama32k,
           W.sweep(B=4, n_k=4096, r=1.0, seed=1003),
           persistent_case((6, 32, 8, 128, 20480, ())),
           W.random_case(2, 8, 2, 128, [3000, 1500], max_n_k=3100, seed=2)]
    probs = [santa.problem(torch.from_numpy(w.q), torch.from_numpy(w.K), w.scale) for w in wls]
    nbytes = max(santa.workspace_bytes(pr) for pr in probs)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    first = [run_decode_det(w, 128, 2, 9, workspace=ws) for w in wls]
    for _ in range(3):
        for w, ref in zip(wls, first):
            _same(run_decode_det(w, 128, 2, 9, workspace=ws), ref)
    # and the first results are the oracle's draw (band rule)
    for w, (out_g, idx_g) in zip(wls[1:], first[1:]):
        out_o, idx_o, det = O.santa_decode(w.q, w.K, w.V, w.n_k, 128, 2, 9, w.scale, return_detail=True)
        rep = P.compare_indices(idx_g, idx_o, det, P.BAND)
        assert rep.bad == 0, rep


def _one_rounding(out_g, idx_g, wl, S):
    """out equals the fp64 estimate on the GPU's own index list (an exact sum
    divided by S) after one rounding to fp32: within half an fp32 ulp of it."""
    est = P.oracle_estimate_from_indices(wl.V, idx_g, wl.n_k, wl.Hq, S)
    valid = (wl.n_k >= 1) & (wl.n_k <= wl.max_n_k)
    e, g = est[valid], out_g[valid].astype(np.float64)
    ulp = np.spacing(np.abs(e).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(g - e) <= 0.5 * ulp + 1e-300), np.abs(g - e).max()


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_deterministic_mode_parity_and_one_rounding(llama32k, mode):
    """The deterministic mode samples the same indices (band rule against the
    oracle) and its output is the exact estimate on those indices, rounded once."""
    wl = llama32k
    S, seed = 128, 61 + mode
    out_g, idx_g = run_decode_det(wl, S, mode, seed)
    out_o, idx_o, det = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale, return_detail=True)
    rep = P.compare_indices(idx_g, idx_o, det, P.BAND)
    print("   deterministic mode %d: %s" % (mode, rep), flush=True)
    assert rep.bad == 0
    _one_rounding(out_g, idx_g, wl, S)


@pytest.mark.parametrize("case", SMALL + PERSISTENT[:1], ids=lambda c: "B%d_Hq%d_Hkv%d_d%d" % c[:4])
def test_deterministic_mode_shapes(case):
    """Head dims 64/128, group sizes 1-8, ragged tails, one split, invalid
    lengths and the persistent variant: exact estimate, rounded once."""
    if len(case) == 6 and isinstance(case[5], tuple):
        wl = persistent_case(case)
    else:
        B, Hq, Hkv, d, n_k, max_n_k = case
        wl = W.random_case(B, Hq, Hkv, d, n_k, max_n_k=max_n_k, seed=71 + B, planted=True,
                           pad_value=np.float16(np.nan))
    for mode, S in ((2, 96), (0, 33)):
        out_g, idx_g = run_decode_det(wl, S, mode, 9)
        valid = (wl.n_k >= 1) & (wl.n_k <= wl.max_n_k)
        assert np.isnan(out_g[~valid]).all()
        _one_rounding(out_g, idx_g, wl, S)
        again = run_decode_det(wl, S, mode, 9)
        assert np.array_equal(np.nan_to_num(again[0]).view(np.uint32), np.nan_to_num(out_g).view(np.uint32))


@pytest.mark.parametrize("mode", [2, 0])
@pytest.mark.parametrize("deterministic", [True, False])
def test_graph_replay_matches_eager(llama32k, mode, deterministic):
    """A captured santa_decode replays correctly, with eager launches on the
    same workspace between replays (the slots are tagged per launch).  In the
    deterministic mode every replay is bit-identical to the eager call."""
    wl = llama32k
    q, K, V, nk = P.to_dev(wl)
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    S = 128
    idx_e = torch.empty((1, 32, S), dtype=torch.int32, device="cuda")
    out_e = santa.santa_decode(q, K, V, nk, S, mode, 42, wl.scale, indices=idx_e, workspace=ws,
                               deterministic=deterministic)
    torch.cuda.synchronize()
    idx_g = torch.empty_like(idx_e)
    out_g = torch.empty_like(out_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        santa.santa_decode(q, K, V, nk, S, mode, 42, wl.scale, out=out_g, indices=idx_g, workspace=ws,
                           deterministic=deterministic)
    for rep in range(4):
        out_g.fill_(7.0)
        idx_g.fill_(-5)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx_e), rep
        if deterministic:
            assert torch.equal(out_g, out_e), rep
        else:
            assert (out_g - out_e).abs().max().item() <= 1e-6, rep
        santa.santa_decode(q, K, V, nk, S, mode, 1000 + rep, wl.scale, workspace=ws,
                           deterministic=deterministic)  # eager work in between
        torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0


# --------------------------------------------------------------------------
# batched long context (B=16, n_k uniform in [8192, 32768]) and the context
# sweep: full-size launches, oracle on sampled heads
# --------------------------------------------------------------------------

def check_sampled_heads(wl, S, mode, seed, heads):
    out_g, idx_g, sc_g = run_decode(wl, S, mode, seed)
    G = wl.Hq // wl.Hkv
    rep = P.IndexReport()
    for (b, h) in heads:
        n = int(wl.n_k[b])
        s = O.head_scores(wl.q[b, h].astype(np.float64), wl.K[b, h // G, :n].astype(np.float64), wl.scale)
        _, _, F = O.distribution(s)
        t = O.points(mode, S, seed, b * wl.Hq + h)
        io = O.inverse_cdf(F, t)
        rep.add(P.compare_head(idx_g[b, h], io, t, F, P.BAND))
        est = O.gather_average(wl.V[b, h // G, :n].astype(np.float64), idx_g[b, h], S)
        assert np.abs(out_g[b, h] - est).max() <= P.OUT_TOL
        assert np.abs(sc_g[b, h, :n] - s).max() <= 1e-4 * max(1.0, np.abs(s).max())
    print("   sampled heads: %s" % rep, flush=True)
    assert rep.bad == 0, rep
    # every head: ascending, in range, finite
    for b in range(wl.B):
        assert np.all(np.diff(idx_g[b], axis=-1) >= 0) and idx_g[b].min() >= 0 and idx_g[b].max() < wl.n_k[b]
    assert np.isfinite(out_g).all()


def test_batched_long_context_sampled():
    wl = W.llama(B=16, n_k_range=(8192, 32768), seed=1002)
    rng = np.random.default_rng(0)
    heads = [(int(b), int(rng.integers(0, 32))) for b in range(16)]
    print("[decode] batched B=16 n_k=%s" % list(wl.n_k), flush=True)
    check_sampled_heads(wl, 128, 2, 77, heads)


@pytest.mark.parametrize("n_k,r", [(4096, 0.5), (16384, 4.0), (65536, 1.0), (131072, 1.0)])
def test_context_sweep_sampled(n_k, r):
    wl = W.sweep(B=4, n_k=n_k, r=r, seed=1003)
    heads = [(0, 0), (1, 7), (2, 19), (3, 31)]
    for mode in (1, 2):
        print("[decode] sweep n_k=%d r=%g mode=%d" % (n_k, r, mode), flush=True)
        check_sampled_heads(wl, 128, mode, 5, heads)


# --------------------------------------------------------------------------
# statistics on the GPU: mean over seeds within 3 sigma of dense attention
# --------------------------------------------------------------------------

def test_gpu_mean_over_seeds_matches_dense():
    from oracle import moments as M
    wl = W.tiny()
    q, K, V, nk = P.to_dev(wl)
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    s = O.head_scores(wl.q[0, 0].astype(np.float64), wl.K[0, 0].astype(np.float64), wl.scale)
    _, _, F = O.distribution(s)
    Vh = wl.V[0, 0].astype(np.float64)
    dense = O.dense_head(s, Vh)
    N, S = 4000, 16
    for mode in (0, 1, 2):
        outs = torch.empty((N, wl.d), dtype=torch.float32, device="cuda")
        for seed in range(N):
            santa.santa_decode(q, K, V, nk, S, mode, seed, wl.scale, out=outs[seed:seed + 1].view(1, 1, wl.d),
                               workspace=ws)
        torch.cuda.synchronize()
        est = outs.cpu().numpy().astype(np.float64)
        _, var = M.moments(mode, F, Vh, S)
        z = (est.mean(axis=0) - dense) / np.sqrt(var / N)
        print("   mode %d: max |z| = %.2f" % (mode, np.abs(z).max()), flush=True)
        assert (np.abs(z) > 3).sum() <= 2 and np.abs(z).max() < 5


def test_iid_many_points_in_one_split_parity():
    # i.i.d. draws where the split holding a heavy key receives several waves'
    # worth (> 128) of the head's points while the other splits keep theirs:
    # the in-range points are packed and searched in rounds of 64
    wl = W.random_case(1, 4, 1, 128, [4096], seed=77, planted=True)
    wl.K[0, 0, 0] = (wl.K[0, 0, 0].astype(np.float32) * 0.7).astype(np.float16)  # sink: about a third of the mass
    S = 512
    for seed in range(3):
        _, idx_o, _ = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, S, 0, seed, wl.scale, return_detail=True)
        in_first = (idx_o[0] < 1024).sum(axis=-1)
        assert in_first.max() > 128 and (idx_o[0] >= 1024).any(), in_first
        check_parity(wl, S, 0, seed, "iid-heavy-split")


def test_stale_exact_sums_never_pass_for_slots(llama32k):
    """The exact sums of a deterministic call carry markers of 2^52 per
    element, so the upper halves of their 64-bit words are launch numbers the
    counters will reach.  Such words left in a shared workspace must never be
    taken for statistics slots of a later launch.  Here the launch counters
    are set so that the next launch number equals the upper half of a stale
    word, and the Llama-layer call must still reproduce, bit for bit, the
    same call on a fresh workspace (deterministic mode)."""
    small = W.random_case(2, 8, 2, 128, [3000, 1500], max_n_k=3100, seed=2, planted=True)
    prob = santa.problem(torch.from_numpy(llama32k.q), torch.from_numpy(llama32k.K), llama32k.scale)
    ws = santa.new_workspace(prob, "cuda")
    run_decode_det(small, 64, 2, 3, workspace=ws)
    words = ws.cpu().numpy().view(np.uint64)
    upper = (words[(1024 + 65536) // 8:] >> np.uint64(32)).astype(np.int64)
    marked = upper[upper >= (1 << 20)]
    assert marked.size > 0  # the exact sums are there
    vals, counts = np.unique(marked, return_counts=True)
    target = int(vals[np.argmax(counts)])
    hdr = words[:128].copy()
    launches = int(sum(int(hdr[16 + 16 * i]) for i in range(7))) >> 20
    assert target > launches + 1  # a launch number not used yet
    hdr[16] = np.uint64((target - 1) << 20)
    for i in range(1, 7):
        hdr[16 + 16 * i] = np.uint64(0)
    ws[:1024].copy_(torch.from_numpy(hdr.view(np.uint8)).to(ws.device))
    got = run_decode_det(llama32k, 128, 2, 11, workspace=ws)
    ref = run_decode_det(llama32k, 128, 2, 11)
    _same(got, ref)
