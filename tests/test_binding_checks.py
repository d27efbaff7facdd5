"""The Python binding rejects wrongly shaped or typed tensors before it calls
the library (which cannot check the size of a device buffer), so a bad call
raises instead of reading or writing out of bounds.  Runs on CPU tensors: every
check fires before any device work."""

import pytest
import torch

from stochastic_sparse_decode_amd import santa

B, HQ, HKV, D, N = 2, 8, 2, 64, 256


def _t(shape, dtype=torch.float16):
    return torch.zeros(shape, dtype=dtype)


def _args(**kw):
    a = dict(q=_t((B, HQ, D)), K=_t((B, HKV, N, D)), V=_t((B, HKV, N, D)), n_k=_t((B,), torch.int32))
    a.update(kw)
    return a


def _decode(**kw):
    a = _args(**{k: v for k, v in kw.items() if k in ("q", "K", "V", "n_k")})
    extra = {k: v for k, v in kw.items() if k not in ("q", "K", "V", "n_k")}
    return santa.santa_decode(a["q"], a["K"], a["V"], a["n_k"], extra.pop("S", 16), 2, 0, 0.125, **extra)


@pytest.mark.parametrize("kw,match", [
    (dict(q=_t((B, HQ))), "q must be"),
    (dict(K=_t((B, HKV, N))), "K must be"),
    (dict(K=_t((B + 1, HKV, N, D))), "K must be"),
    (dict(K=_t((B, 3, N, D))), "multiple of H_kv"),
    (dict(V=_t((B, HKV, N - 1, D))), "V must have shape"),
    (dict(n_k=_t((B + 1,), torch.int32)), "n_k must have shape"),
    (dict(out=_t((B, HQ, D + 1), torch.float32)), "out must have shape"),
    (dict(indices=_t((B, HQ, 15), torch.int32)), "indices must have shape"),
    (dict(scores=_t((B, HQ, N - 64), torch.float32)), "scores must have shape"),
])
def test_santa_decode_rejects_bad_shapes(kw, match):
    with pytest.raises(ValueError, match=match):
        _decode(**kw)


def test_santa_decode_rejects_bad_dtypes_and_cpu_tensors():
    with pytest.raises(TypeError):
        _decode(V=_t((B, HKV, N, D), torch.float32))
    with pytest.raises(TypeError):
        _decode(n_k=_t((B,), torch.int64))
    with pytest.raises(ValueError, match="contiguous"):
        _decode(K=_t((B, HKV, D, N)).transpose(2, 3))
    with pytest.raises(ValueError, match="GPU"):
        _decode()  # every shape right: only the device is wrong


def test_workspace_size_is_checked():
    a = _args()
    with pytest.raises(ValueError):
        santa._check_workspace(torch.zeros(16, dtype=torch.uint8), santa.problem(a["q"], a["K"], 0.125),
                               torch.device("cpu"))


def test_fp8k_paged_bernoulli_dense_shapes():
    a = _args()
    with pytest.raises(ValueError, match="k_scale must have shape"):
        santa.santa_decode_fp8k(a["q"], _t((B, HKV, N, D), torch.uint8), _t((B,), torch.float32), a["V"], a["n_k"],
                                16, 2, 0, 0.125)
    with pytest.raises(TypeError):
        santa.santa_decode_fp8k(a["q"], a["K"], _t((B, HKV), torch.float32), a["V"], a["n_k"], 16, 2, 0, 0.125)
    kc = _t((10, HKV, 64, D))
    with pytest.raises(ValueError, match="block_table must be"):
        santa.santa_decode_paged(a["q"], kc, kc, _t((B + 1, 4), torch.int32), a["n_k"], 16, 2, 0, 0.125)
    with pytest.raises(ValueError, match="V_cache must have shape"):
        santa.santa_decode_paged(a["q"], kc, _t((10, HKV, 32, D)), _t((B, 4), torch.int32), a["n_k"], 16, 2, 0,
                                 0.125)
    kfm = _t((B, HKV, N // 64, D, 64))
    with pytest.raises(ValueError, match="K_fm must be"):
        santa.santa_bernoulli_qk(a["q"], _t((B, HKV, N // 64, D, 32)), a["V"], a["n_k"], 16, 2, 0, 0.125)
    with pytest.raises(ValueError, match="kept must have shape"):
        santa.santa_bernoulli_qk(a["q"], kfm, a["V"], a["n_k"], 16, 2, 0, 0.125, kept=_t((B, HQ, D - 1), torch.uint8))
    with pytest.raises(ValueError, match="out must have shape"):
        santa.santa_dense_decode(a["q"], a["K"], a["V"], a["n_k"], 0.125, out=_t((B, HQ, 2 * D), torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        santa.santa_dense_decode(a["q"], a["K"], a["V"], a["n_k"], 0.125)
