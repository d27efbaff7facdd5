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
