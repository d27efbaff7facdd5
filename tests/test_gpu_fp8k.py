"""GPU parity of santa_decode_fp8k (fp8 E4M3 key cache) against the fp64
oracle, through the C-ABI.  Same bars as the fp16 path: indices bit-exact
except for points within 1e-5 of a separating CDF value (and within 1e-6 when
the oracle reruns on the GPU's own scores), outputs within 2e-3, scores within
1e-4 relative of the oracle's fp64 scores on the exactly decoded keys."""

import functools

import numpy as np
import pytest
import torch

from oracle import fp8, santa as O
from stochastic_sparse_decode_amd import santa
from stochastic_sparse_decode_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def fp8_case(wl):
    K8, ks = W.quantize_keys_fp8(wl.K, wl.n_k)
    return K8, ks


def run_fp8k(wl, K8, ks, S, mode, seed, workspace=None, with_scores=True):
    q, _, V, nk = P.to_dev(wl)
    K8d = torch.from_numpy(K8).cuda()
    ksd = torch.from_numpy(ks).cuda()
    B, Hq = wl.B, wl.Hq
    idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((B, Hq, wl.max_n_k), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
    ws = workspace if workspace is not None else santa.new_workspace(santa.problem(q, K8d, wl.scale), q.device)
    out = santa.santa_decode_fp8k(q, K8d, ksd, V, nk, S, mode, seed, wl.scale, indices=idx, scores=sc,
                                  workspace=ws)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0
    return out.cpu().numpy(), idx.cpu().numpy(), (sc.cpu().numpy() if sc is not None else None)


def check_fp8k(wl, K8, ks, S, mode, seed, label=""):
    print("[fp8k] %s S=%d mode=%d seed=%d B=%d Hq=%d Hkv=%d d=%d n_k=%s" % (
        label, S, mode, seed, wl.B, wl.Hq, wl.Hkv, wl.d, list(wl.n_k)[:4]), flush=True)
    out_g, idx_g, sc_g = run_fp8k(wl, K8, ks, S, mode, seed)
    out_o, idx_o, det = O.santa_decode_fp8k(wl.q, K8, ks, wl.V, wl.n_k, S, mode, seed, wl.scale,
                                            return_detail=True)
    valid = (wl.n_k >= 1) & (wl.n_k <= wl.max_n_k)
    assert np.isnan(out_g[~valid]).all() and (idx_g[~valid] == -1).all()
    for b in np.nonzero(valid)[0]:
        assert np.all(np.diff(idx_g[b], axis=-1) >= 0)
        assert idx_g[b].min() >= 0 and idx_g[b].max() < wl.n_k[b]
    flips = set()
    rep = P.compare_indices(idx_g, idx_o, det, P.BAND, flips)
    _, idx_s, det_s = O.santa_decode_fp8k(wl.q, K8, ks, wl.V, wl.n_k, S, mode, seed, wl.scale,
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
    s_o = O.all_scores(wl.q, fp8.dequantize(K8, ks), wl.n_k, wl.scale)
    m = ~np.isnan(s_o)
    assert np.abs(sc_g[m] - s_o[m]).max() <= 1e-4 * max(1.0, np.abs(s_o[m]).max())


SMALL = [
    # B, Hq, Hkv, d, n_k, max_n_k
    (2, 8, 2, 128, [3000, 1500], 3100),
    (1, 16, 2, 128, [4500], 4500),
    (1, 4, 4, 128, [2049], 2049),
    (3, 8, 2, 64, [777, 2048, 1025], 2100),
    (2, 2, 1, 64, [1024, 1], 1024),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%d_Hq%d_Hkv%d_d%d" % c[:4])
@pytest.mark.parametrize("mode", [2, 1, 0])
def test_fp8k_small_shapes_parity(case, mode):
    B, Hq, Hkv, d, n_k, max_n_k = case
    wl = W.random_case(B, Hq, Hkv, d, n_k, max_n_k=max_n_k, seed=41 + B + d, planted=True,
                       pad_value=np.float16(np.nan))
    K8, ks = fp8_case(wl)
    for S in (8, 128):
        check_fp8k(wl, K8, ks, S, mode, 200 + S, "small")


def test_fp8k_invalid_lengths():
    wl = W.random_case(3, 8, 2, 128, [0, 1200, 5000], max_n_k=2048, seed=6)
    K8, ks = fp8_case(wl)
    check_fp8k(wl, K8, ks, 16, 2, 3, "invalid-n_k")


@functools.lru_cache(maxsize=1)
def llama32k_fp8():
    wl = W.llama(B=1, n_k=32768, seed=1001)
    return wl, fp8_case(wl)


@pytest.mark.parametrize("mode", [2, 1, 0])
@pytest.mark.parametrize("S", [32, 128])
def test_fp8k_llama32k_parity(mode, S):
    wl, (K8, ks) = llama32k_fp8()
    check_fp8k(wl, K8, ks, S, mode, 1 + S, "llama32k")


@functools.lru_cache(maxsize=1)
def persistent_fp8():
    B, max_n_k = 20, 16384
    rng = np.random.default_rng(91)
    n_k = rng.integers(1, max_n_k + 1, size=B).astype(np.int32)
    n_k[2], n_k[13] = 0, max_n_k + 1
    wl = W.random_case(B, 32, 8, 128, n_k, max_n_k=max_n_k, seed=92, planted=True, pad_value=np.float16(np.nan))
    return wl, fp8_case(wl)


@pytest.mark.parametrize("mode", [2, 1, 0])
def test_fp8k_persistent_ragged_invalid_parity(mode):
    wl, (K8, ks) = persistent_fp8()
    assert wl.B * wl.Hkv * (wl.max_n_k // 1024) > 2048
    check_fp8k(wl, K8, ks, 32, mode, 17, "persistent")


def test_fp8k_matches_fp16_path_on_decoded_keys():
    """With k_scale = 1 and keys given as the fp16 values of the fp8 codes, the
    fp8 and fp16 steps compute the same scores up to fp32 summation order."""
    wl = W.random_case(2, 8, 2, 128, [2500, 900], max_n_k=2560, seed=8)
    K8, _ = fp8_case(wl)
    ones = np.ones((wl.B, wl.Hkv), dtype=np.float32)
    out8, idx8, sc8 = run_fp8k(wl, K8, ones, 64, 2, 5)
    wl.K[:] = fp8.decode(K8).astype(np.float16)  # exact: E4M3 values are fp16 values
    q, K, V, nk = P.to_dev(wl)
    sc = torch.full((wl.B, wl.Hq, wl.max_n_k), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.B, wl.Hq, 64), dtype=torch.int32, device="cuda")
    santa.santa_decode(q, K, V, nk, 64, 2, 5, wl.scale, indices=idx, scores=sc)
    torch.cuda.synchronize()
    sc = sc.cpu().numpy()
    m = ~np.isnan(sc)
    assert np.abs(sc8[m] - sc[m]).max() <= 1e-5 * max(1.0, np.abs(sc[m]).max())
    # both steps sample the oracle's indices on the decoded keys (up to the band)
    _, idx_o, det = O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, 64, 2, 5, wl.scale, return_detail=True)
    for got in (idx8, idx.cpu().numpy()):
        rep = P.compare_indices(got, idx_o, det, P.BAND)
        print("   %s" % rep, flush=True)
        assert rep.bad == 0, rep
