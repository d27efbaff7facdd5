"""Pins for the oracle's paged-cache gather and paged decode driver (CPU)."""

import numpy as np

from oracle import santa
from stochastic_sparse_decode_amd import workloads as W


def _paginate_by_hand(K, n_k, P, order):
    """Independent construction: blocks listed sequence by sequence, stored
    at the positions ``order`` gives them."""
    B, Hkv, _, d = K.shape
    blocks = []
    for b in range(B):
        for i in range((int(n_k[b]) + P - 1) // P):
            blocks.append((b, i))
    cache = np.zeros((len(blocks), Hkv, P, d), dtype=np.float16)
    table = np.full((B, (K.shape[2] + P - 1) // P), -1, dtype=np.int32)
    for (b, i), pos in zip(blocks, order):
        rows = min(P, int(n_k[b]) - i * P)
        for h in range(Hkv):
            for r in range(rows):
                cache[pos, h, r] = K[b, h, i * P + r]
        table[b, i] = pos
    return cache, table


def test_gather_inverts_an_independent_pagination():
    wl = W.random_case(3, 4, 2, 64, [70, 16, 33], max_n_k=80, seed=3)
    P = 16
    nblk = sum((int(n) + P - 1) // P for n in wl.n_k)
    order = np.random.default_rng(4).permutation(nblk)
    cache, table = _paginate_by_hand(wl.K, wl.n_k, P, order)
    got = santa.gather_paged(cache, table, wl.n_k, wl.max_n_k)
    for b in range(3):
        n = int(wl.n_k[b])
        assert np.array_equal(got[b, :, :n], wl.K[b, :, :n].astype(np.float64))
        assert np.isnan(got[b, :, n:]).all()


def test_paged_step_equals_contiguous_step():
    wl = W.random_case(2, 8, 2, 64, [300, 97], max_n_k=320, seed=5, planted=True)
    for P in (16, 64):
        Kc, Vc, table, nb = W.paginate(wl.K, wl.V, wl.n_k, P, seed=P)
        assert table.max() < nb
        for mode in (0, 1, 2):
            o1, i1 = santa.santa_decode_paged(wl.q, Kc, Vc, table, wl.n_k, wl.max_n_k, 32, mode, 9, wl.scale)
            o2, i2 = santa.santa_decode(wl.q, wl.K, wl.V, wl.n_k, 32, mode, 9, wl.scale)
            assert np.array_equal(i1, i2)
            assert np.array_equal(o1, o2)


def test_paged_bad_block_or_length_gives_nan():
    wl = W.random_case(3, 4, 2, 64, [100, 50, 20], max_n_k=128, seed=6)
    Kc, Vc, table, nb = W.paginate(wl.K, wl.V, wl.n_k, 32, seed=1)
    table = table.copy()
    table[1, 0] = nb          # out of range
    n_k = wl.n_k.copy()
    n_k[2] = 0                # invalid length
    o, i = santa.santa_decode_paged(wl.q, Kc, Vc, table, n_k, wl.max_n_k, 8, 2, 1, wl.scale)
    assert not np.isnan(o[0]).any() and (i[0] >= 0).all()
    assert np.isnan(o[1]).all() and (i[1] == -1).all()
    assert np.isnan(o[2]).all() and (i[2] == -1).all()
