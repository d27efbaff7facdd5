"""GPU parity of santa_dense_decode (exact split-K attention) against the oracle."""

import numpy as np
import pytest
import torch

from oracle import santa as O
from stochastic_sparse_decode_amd import santa
from stochastic_sparse_decode_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def run_dense(wl):
    q, K, V, nk = P.to_dev(wl)
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    out = santa.santa_dense_decode(q, K, V, nk, wl.scale, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    ("tiny", lambda: W.tiny()),
    ("gqa4_ragged", lambda: W.random_case(2, 8, 2, 128, [3000, 1500], max_n_k=3100, seed=3, planted=True,
                                          pad_value=np.float16(np.nan))),
    ("d64_g2", lambda: W.random_case(3, 4, 2, 64, [1, 1030, 2048], max_n_k=2048, seed=4)),
    ("g8", lambda: W.random_case(1, 16, 2, 128, [5000], seed=6, planted=True)),
    ("g1_d128", lambda: W.random_case(2, 4, 4, 128, [3000, 777], max_n_k=3072, seed=9, planted=True)),
    ("llama32k", lambda: W.llama(B=1, n_k=32768, seed=1001)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_dense_parity(name, make):
    wl = make()
    print("[dense] %s B=%d Hq=%d Hkv=%d d=%d n_k=%s" % (name, wl.B, wl.Hq, wl.Hkv, wl.d, list(wl.n_k)), flush=True)
    got = run_dense(wl)
    ref = O.dense_decode(wl.q, wl.K, wl.V, wl.n_k, wl.scale)
    err = np.abs(got - ref).max()
    print("   max abs err %.3g" % err, flush=True)
    assert err <= P.DENSE_TOL


def test_dense_batched_sampled_heads():
    wl = W.llama(B=16, n_k_range=(8192, 32768), seed=1002)
    got = run_dense(wl)
    G = wl.Hq // wl.Hkv
    for b in range(16):
        h = (5 * b + 3) % 32
        n = int(wl.n_k[b])
        s = O.head_scores(wl.q[b, h].astype(np.float64), wl.K[b, h // G, :n].astype(np.float64), wl.scale)
        ref = O.dense_head(s, wl.V[b, h // G, :n].astype(np.float64))
        assert np.abs(got[b, h] - ref).max() <= P.DENSE_TOL
    assert np.isfinite(got).all()


def test_dense_invalid_lengths_are_nan():
    wl = W.random_case(2, 4, 2, 128, [0, 100], max_n_k=128, seed=8)
    got = run_dense(wl)
    assert np.isnan(got[0]).all() and np.isfinite(got[1]).all()


# Every item resident at once: the splits of a KV head exchange tagged records
# and each merges a share of the features.  Many splits (64 and 128, the most
# the exchange takes), one KV head per group (G = 1 at d = 64), shares that
# straddle two heads (6 splits of 512 features).
EXCH_CASES = [
    ("nsg64", lambda: W.random_case(1, 32, 8, 128, [65536], seed=21)),
    ("nsg128_g8", lambda: W.random_case(1, 16, 2, 128, [131072 - 700], max_n_k=131072, seed=22, planted=True)),
    ("g1_d64", lambda: W.random_case(2, 8, 8, 64, [7000, 333], max_n_k=7168, seed=23)),
]


@pytest.mark.parametrize("name,make", EXCH_CASES, ids=[c[0] for c in EXCH_CASES])
def test_dense_exchange_parity(name, make):
    wl = make()
    print("[dense exchange] %s B=%d Hq=%d Hkv=%d d=%d n_k=%s" % (name, wl.B, wl.Hq, wl.Hkv, wl.d, list(wl.n_k)),
          flush=True)
    got = run_dense(wl)
    ref = O.dense_decode(wl.q, wl.K, wl.V, wl.n_k, wl.scale)
    err = np.abs(got - ref).max()
    print("   max abs err %.3g" % err, flush=True)
    assert err <= P.DENSE_TOL


def _launch_count(ws):
    """Sum of the workspace's launch counters (7 words, one per 128 bytes from byte 128)."""
    words = ws[:1024].cpu().numpy().view(np.uint64)
    return int(sum(int(words[16 + 16 * i]) for i in range(7)))


def test_dense_exchange_tags_and_repeats():
    """One workspace serves exchange launches of different shapes, a
    persistent dense launch and a sampling launch in turn.  Each exchange
    launch advances the launch count by exactly one unit (2^20), accepts no
    record of an earlier launch, and repeats its first output bit for bit."""
    wls = [W.random_case(1, 32, 8, 128, [20000], max_n_k=20480, seed=31),
           W.random_case(2, 8, 2, 128, [3000, 1500], max_n_k=3100, seed=32, planted=True),
           W.random_case(1, 32, 8, 128, [18000], max_n_k=20480, seed=33)]
    batched = W.llama(B=16, n_k_range=(2048, 8192), seed=34)
    probs = [santa.problem(torch.from_numpy(w.q), torch.from_numpy(w.K), w.scale) for w in wls + [batched]]
    ws = torch.zeros(max(santa.workspace_bytes(pr) for pr in probs), dtype=torch.uint8, device="cuda")
    dev = [P.to_dev(w) for w in wls]

    def dense(i):
        q, K, V, nk = dev[i]
        before = _launch_count(ws)
        out = santa.santa_dense_decode(q, K, V, nk, wls[i].scale, workspace=ws)
        torch.cuda.synchronize()
        assert _launch_count(ws) - before == 1 << 20
        assert santa.santa_workspace_error(ws) == 0
        return out.cpu().numpy()

    first = [dense(i) for i in range(len(wls))]
    for w, got in zip(wls, first):
        ref = O.dense_decode(w.q, w.K, w.V, w.n_k, w.scale)
        assert np.abs(got - ref).max() <= P.DENSE_TOL
    qb, Kb, Vb, nkb = P.to_dev(batched)
    for rep in range(2):
        for i in (2, 0, 1):
            assert np.array_equal(dense(i).view(np.uint32), first[i].view(np.uint32)), (rep, i)
        # a persistent dense launch (float records, no tag) and a sampling launch in between
        santa.santa_dense_decode(qb, Kb, Vb, nkb, batched.scale, workspace=ws)
        q, K, V, nk = dev[1]
        santa.santa_decode(q, K, V, nk, 64, 2, 5 + rep, wls[1].scale, workspace=ws)
        torch.cuda.synchronize()
        assert santa.santa_workspace_error(ws) == 0


def test_dense_exchange_mixed_groups_in_one_launch():
    """One resident launch whose groups take every exchange case: an invalid
    length (NaN rows), one split (the output written directly), two splits
    and eighteen (shares straddling heads)."""
    wl = W.random_case(4, 8, 2, 128, [0, 300, 700, 9000], max_n_k=9216, seed=41, planted=True)
    got = run_dense(wl)
    assert np.isnan(got[0]).all()
    for b in range(1, 4):
        n = int(wl.n_k[b])
        ref = O.dense_decode(wl.q[b:b + 1], wl.K[b:b + 1, :, :n], wl.V[b:b + 1, :, :n], wl.n_k[b:b + 1], wl.scale)
        err = np.abs(got[b] - ref[0]).max()
        print("   b=%d n_k=%d max abs err %.3g" % (b, n, err), flush=True)
        assert err <= P.DENSE_TOL
