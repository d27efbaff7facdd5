"""GPU parity of santa_decode_paged (block-table KV cache) against the fp64
oracle, through the C-ABI.  Same bars as the contiguous path; the cache pools
are built by a seeded paginator with shuffled block placement, NaN in spare
blocks and past each sequence's last key (a read of them poisons the
result)."""

import functools

import numpy as np
import pytest
import torch

from oracle import santa as O
from stochastic_sparse_decode_amd import santa
from stochastic_sparse_decode_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def run_paged(wl, cache, S, mode, seed, expect_err=0, with_scores=True):
    Kc, Vc, table, _ = cache
    q = torch.from_numpy(wl.q).cuda()
    nk = torch.from_numpy(wl.n_k.astype(np.int32)).cuda()
    Kd, Vd, Td = torch.from_numpy(Kc).cuda(), torch.from_numpy(Vc).cuda(), torch.from_numpy(table).cuda()
    B, Hq = wl.B, wl.Hq
    idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hq, wl.max_n_k), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    ws = santa.new_workspace(santa.problem_paged(q, Kd, Td, wl.scale), q.device)
    out = santa.santa_decode_paged(q, Kd, Vd, Td, nk, S, mode, seed, wl.scale, indices=idx, scores=sc, workspace=ws)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == expect_err
    return out.cpu().numpy(), idx.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def check_paged(wl, cache, S, mode, seed, label=""):
    Kc, Vc, table, _ = cache
    print("[paged] %s P=%d S=%d mode=%d B=%d Hq=%d Hkv=%d d=%d n_k=%s" % (
        label, Kc.shape[2], S, mode, wl.B, wl.Hq, wl.Hkv, wl.d, list(wl.n_k)[:4]), flush=True)
    out_g, idx_g, sc_g = run_paged(wl, cache, S, mode, seed)
    out_o, idx_o, det = O.santa_decode_paged(wl.q, Kc, Vc, table, wl.n_k, wl.max_n_k, S, mode, seed, wl.scale,
                                             return_detail=True)
    valid = (wl.n_k >= 1) & (wl.n_k <= wl.max_n_k)
    assert np.isnan(out_g[~valid]).all() and (idx_g[~valid] == -1).all()
    for b in np.nonzero(valid)[0]:
        assert np.all(np.diff(idx_g[b], axis=-1) >= 0)
        assert idx_g[b].min() >= 0 and idx_g[b].max() < wl.n_k[b]
    flips = set()
    rep = P.compare_indices(idx_g, idx_o, det, P.BAND, flips)
    _, idx_s, det_s = O.santa_decode_paged(wl.q, Kc, Vc, table, wl.n_k, wl.max_n_k, S, mode, seed, wl.scale,
                                           score_override=sc_g, return_detail=True)
    rep2 = P.compare_indices(idx_g, idx_s, det_s, P.BAND_SAME_SCORES)
    print("   vs oracle: %s | on GPU scores: %s" % (rep, rep2), flush=True)
    assert rep.bad == 0, rep
    assert rep2.bad == 0, rep2
    est = P.oracle_estimate_from_indices(wl.V, idx_g, wl.n_k, wl.Hq, S)
    assert np.abs(out_g[valid] - est[valid]).max() <= P.OUT_TOL
    for b in np.nonzero(valid)[0]:
        for h in range(wl.Hq):
            if (b, h) not in flips:
                assert np.abs(out_g[b, h] - out_o[b, h]).max() <= P.OUT_TOL
    s_o = O.all_scores(wl.q, wl.K, wl.n_k, wl.scale)
    m = ~np.isnan(s_o)
    assert np.abs(sc_g[m] - s_o[m]).max() <= 1e-4 * max(1.0, np.abs(s_o[m]).max())


SMALL = [
    # B, Hq, Hkv, d, n_k, max_n_k, block size
    (2, 8, 2, 128, [3000, 1500], 3072, 16),
    (3, 8, 2, 64, [777, 2048, 1025], 2560, 64),
    (1, 16, 2, 128, [4500], 4608, 256),
    (2, 4, 4, 128, [2049, 100], 3072, 1024),
    (2, 2, 1, 64, [1024, 1], 1024, 32),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d_P%d" % (c[:4] + (c[6],)))
@pytest.mark.parametrize("mode", [2, 1, 0])
def test_paged_small_shapes_parity(case, mode):
    B, Hq, Hkv, d, n_k, max_n_k, blk = case
    wl = W.random_case(B, Hq, Hkv, d, n_k, max_n_k=max_n_k, seed=51 + B + d, planted=True,
                       pad_value=np.float16(np.nan))
    cache = W.paginate(wl.K, wl.V, wl.n_k, blk, seed=blk)
    for S in (8, 128):
        check_paged(wl, cache, S, mode, 300 + S, "small")


@functools.lru_cache(maxsize=1)
def llama32k():
    return W.llama(B=1, n_k=32768, seed=1001)


@pytest.mark.parametrize("blk", [16, 256])
@pytest.mark.parametrize("mode", [2, 0])
def test_paged_llama32k_parity(blk, mode):
    wl = llama32k()
    check_paged(wl, W.paginate(wl.K, wl.V, wl.n_k, blk, seed=7), 128, mode, 5, "llama32k")


@functools.lru_cache(maxsize=1)
def persistent_case():
    B, max_n_k = 20, 16384
    rng = np.random.default_rng(93)
    n_k = rng.integers(1, max_n_k + 1, size=B).astype(np.int32)
    n_k[4], n_k[17] = 0, max_n_k + 1
    wl = W.random_case(B, 32, 8, 128, n_k, max_n_k=max_n_k, seed=94, planted=True, pad_value=np.float16(np.nan))
    return wl, W.paginate(wl.K, wl.V, wl.n_k, 128, seed=95)


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_paged_persistent_ragged_invalid_parity(mode):
    wl, cache = persistent_case()
    assert wl.B * wl.Hkv * (wl.max_n_k // 1024) > 2048
    check_paged(wl, cache, 32, mode, 17, "persistent")


def test_paged_block_entry_out_of_range_sets_error_bit():
    """An entry outside the pool is read as block 0 (no fault) and reported;
    the other sequences are unaffected."""
    wl = W.random_case(3, 8, 2, 128, [900, 1500, 700], max_n_k=2048, seed=12)
    Kc, Vc, table, nb = W.paginate(wl.K, wl.V, wl.n_k, 64, seed=3)
    bad = table.copy()
    bad[1, 3] = nb + 5
    out_g, idx_g, _ = run_paged(wl, (Kc, Vc, bad, nb), 16, 2, 4, expect_err=2)
    out_o, idx_o, det = O.santa_decode_paged(wl.q, Kc, Vc, table, wl.n_k, wl.max_n_k, 16, 2, 4, wl.scale,
                                             return_detail=True)
    flips = set()
    rep = P.IndexReport()
    for b in (0, 2):
        rep.add(P.compare_indices(idx_g[b:b + 1], idx_o[b:b + 1],
                                  {"t": {(0, h): det["t"][(b, h)] for h in range(wl.Hq)},
                                   "F": {(0, h): det["F"][(b, h)] for h in range(wl.Hq)}}, P.BAND, flips))
        est = P.oracle_estimate_from_indices(wl.V[b:b + 1], idx_g[b:b + 1], wl.n_k[b:b + 1], wl.Hq, 16)
        assert np.abs(out_g[b] - est[0]).max() <= P.OUT_TOL
        for h in range(wl.Hq):
            if (0, h) not in flips:
                assert np.abs(out_g[b, h] - out_o[b, h]).max() <= P.OUT_TOL
        flips.clear()
    print("   unaffected sequences: %s" % rep, flush=True)
    assert rep.bad == 0, rep
