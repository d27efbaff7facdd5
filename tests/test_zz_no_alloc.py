"""The allocation-free entry point (santa_decode_noalloc) against santa_decode.

It runs the same computation on the library's own workspace: the sampled
indices must equal santa_decode's bit for bit and the outputs must agree to the
output tolerance (bit for bit in the deterministic mode), on two calls in a row
where the second has a smaller input (the array keeps the first call's
contents).  A problem beyond the array's size is rejected."""

import ctypes

import numpy as np
import pytest
import torch

from stochastic_sparse_decode_amd import santa
from stochastic_sparse_decode_amd import workloads as W
from tests import parity as P

pytestmark = pytest.mark.gpu


def _pair(wl, S, mode, seed, deterministic):
    q, K, V, nk = P.to_dev(wl)
    idx_a = torch.full((wl.B, wl.Hq, S), -7, dtype=torch.int32, device="cuda")
    idx_b = torch.full_like(idx_a, -9)
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), q.device)
    out_a = santa.santa_decode(q, K, V, nk, S, mode, seed, wl.scale, indices=idx_a, workspace=ws,
                               deterministic=deterministic)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out_b = santa.santa_decode_noalloc(q, K, V, nk, S, mode, seed, wl.scale, indices=idx_b, error_flags=err,
                                       deterministic=deterministic)
    torch.cuda.synchronize()
    assert santa.santa_workspace_error(ws) == 0
    assert int(err.item()) == 0
    return out_a.cpu().numpy(), idx_a.cpu().numpy(), out_b.cpu().numpy(), idx_b.cpu().numpy()


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("mode", [2, 0])
def test_noalloc_matches_santa_decode_on_two_calls(mode, deterministic):
    big = W.llama(B=1, n_k=32768, seed=1001)
    small = W.random_case(2, 8, 2, 128, [3000, 1500], max_n_k=3100, seed=2, planted=True,
                          pad_value=np.float16(np.nan))
    for wl, S, seed in ((big, 128, 3), (small, 64, 4)):  # the second call is smaller
        out_a, idx_a, out_b, idx_b = _pair(wl, S, mode, seed, deterministic)
        assert np.array_equal(idx_a, idx_b)
        if deterministic:
            assert np.array_equal(out_a.view(np.uint32), out_b.view(np.uint32))
        else:
            assert np.abs(out_a - out_b).max() <= P.OUT_TOL
            # both match the oracle's estimate on the common index list
            est = P.oracle_estimate_from_indices(wl.V, idx_b, wl.n_k, wl.Hq, S)
            assert np.abs(out_b - est).max() <= P.OUT_TOL


def test_noalloc_rejects_a_problem_beyond_its_array():
    lib = santa.library()
    prob = santa.Problem(512, 32, 8, 128, 1 << 20, 0.125, 0)  # sampling workspace far above 16 MiB
    vp = ctypes.c_void_p
    assert lib.santa_decode_noalloc(ctypes.byref(prob), vp(16), vp(16), vp(16), vp(16), 8, 2, 0, vp(16), None,
                                    None, None, None) == 5
