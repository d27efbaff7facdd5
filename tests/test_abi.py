"""The C-ABI library loads, exports what include/santa.h declares, and rejects
bad arguments on the host before any HIP call (runs without a GPU)."""

import ctypes
import os
import re

import pytest

from stochastic_sparse_decode_amd import santa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "santa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(santa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return santa.library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 8
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert santa.santa_abi_version() == 3
    for code in range(8):
        assert santa.status_string(code).startswith("SANTA_")
    assert "unknown" in santa.status_string(99)


def _prob(**kw):
    p = dict(batch=1, num_q_heads=32, num_kv_heads=8, head_dim=128, max_n_k=32768, scale=0.125, flags=0)
    p.update(kw)
    return santa.Problem(**p)


def test_workspace_bytes(lib):
    n = santa.workspace_bytes(_prob())
    # 8 groups x 32 splits x 4 heads x (128 + 2) floats of partials at least
    assert n >= 8 * 32 * 4 * 130 * 4
    assert santa.workspace_bytes(_prob(num_q_heads=30)) == 0  # not a multiple of H_kv
    assert santa.workspace_bytes(_prob(batch=0)) == 0
    assert santa.workspace_bytes(_prob(scale=float("inf"))) == 0
    # the sample count sizes the Gumbel-max winners (B * H_q * S words)
    assert santa.workspace_bytes(_prob(), 0) == 0 and santa.workspace_bytes(_prob(), santa.MAX_S + 1) == 0
    short = _prob(batch=8, max_n_k=1024)  # the sampling layout (with the winners) dominates here
    assert santa.workspace_bytes(short, 1024) - santa.workspace_bytes(short, 1) >= 8 * 32 * 1023 * 8


FAKE = 0x10000  # never dereferenced: every call below fails its host checks


def _decode(lib, prob, S=128, mode=2, q=FAKE, K=FAKE, V=FAKE, nk=FAKE, out=FAKE, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = santa.workspace_bytes(prob) if santa.workspace_bytes(prob) else 1 << 30
    vp = ctypes.c_void_p
    return lib.santa_decode(ctypes.byref(prob), vp(q), vp(K), vp(V), vp(nk), S, mode, 0, vp(out), None, None,
                            vp(ws), ws_bytes, None)


def test_host_checks_return_status_without_touching_the_gpu(lib):
    p = _prob()
    assert lib.santa_decode(None, None, None, None, None, 1, 2, 0, None, None, None, None, 0, None) == 1
    assert _decode(lib, p, q=0) == 1                       # NULL q
    assert _decode(lib, _prob(num_q_heads=30)) == 2        # H_q % H_kv
    assert _decode(lib, _prob(head_dim=96)) == 3           # unsupported d
    assert _decode(lib, _prob(num_q_heads=24, num_kv_heads=8)) == 3  # G = 3
    assert _decode(lib, p, K=FAKE + 8) == 4                # misaligned K
    assert _decode(lib, p, ws_bytes=16) == 5               # workspace too small
    assert _decode(lib, p, ws=0) == 5
    assert _decode(lib, p, S=0) == 2
    assert _decode(lib, p, S=santa.MAX_S + 1) == 2
    assert _decode(lib, p, mode=4) == 7
    assert _decode(lib, p, mode=-1) == 7
    vp = ctypes.c_void_p
    # Bernoulli needs max_n_k % 64 == 0
    pb = _prob(max_n_k=1000)
    assert lib.santa_bernoulli_qk(ctypes.byref(pb), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 8, 2, 0, vp(FAKE),
                                  None, None, None, vp(FAKE), santa.workspace_bytes(pb), None) == 2
    assert lib.santa_pack_k_feature_major(ctypes.byref(pb), vp(FAKE), vp(FAKE), None) == 2
    assert lib.santa_dense_decode(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(0), vp(FAKE),
                                  santa.workspace_bytes(p), None) == 1
    assert lib.santa_workspace_error(None, None, None) == 1


def test_binding_has_no_fallback(tmp_path, monkeypatch):
    monkeypatch.setattr(santa, "_lib", None)
    monkeypatch.setattr(santa, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        santa.library()


def test_fp8k_host_checks(lib):
    vp = ctypes.c_void_p
    p = _prob()
    nb = santa.workspace_bytes(p)

    def call(prob, k_scale, ws_bytes=nb):
        return lib.santa_decode_fp8k(ctypes.byref(prob), vp(FAKE), vp(FAKE), vp(k_scale), vp(FAKE), vp(FAKE), 128,
                                     2, 0, vp(FAKE), None, None, vp(FAKE), ws_bytes, None)

    assert call(p, 0) == 1                     # k_scale missing
    assert call(p, FAKE + 2) == 4              # k_scale not 4-byte aligned
    p64 = _prob(head_dim=64, num_q_heads=64, num_kv_heads=8)
    assert call(p64, FAKE, santa.workspace_bytes(p64)) == 3   # d = 64 with G = 8 is not built
    assert call(p, FAKE, 16) == 5              # workspace too small
    assert lib.santa_decode_fp8k(ctypes.byref(p), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 128, 3, 0,
                                 vp(FAKE), None, None, vp(FAKE), nb, None) == 3  # Gumbel draws: santa_decode only


def test_paged_host_checks(lib):
    vp = ctypes.c_void_p
    p = _prob(max_n_k=4096)
    nb = santa.workspace_bytes(p)

    def call(prob, table=FAKE, block=64, blocks=10, ws_bytes=nb):
        return lib.santa_decode_paged(ctypes.byref(prob), vp(FAKE), vp(FAKE), vp(FAKE), vp(table), block, blocks,
                                      vp(FAKE), 128, 2, 0, vp(FAKE), None, None, vp(FAKE), ws_bytes, None)

    assert call(p, table=0) == 1          # block table missing
    assert call(p, table=FAKE + 2) == 4   # block table not 4-byte aligned
    assert call(p, block=48) == 2         # not a power of two
    assert call(p, block=8) == 2          # below 16 keys
    assert call(p, block=2048) == 2       # above one split
    assert call(_prob(max_n_k=4000), block=64, ws_bytes=santa.workspace_bytes(_prob(max_n_k=4000))) == 2
    assert call(p, blocks=0) == 2         # empty pool
    assert call(p, ws_bytes=16) == 5


def test_bernoulli_budget_host_checks(lib):
    vp = ctypes.c_void_p
    p = _prob()
    nb = santa.workspace_bytes(p)

    def call(budget, prob=p):
        return lib.santa_bernoulli_qk_budget(ctypes.byref(prob), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 8, 2, 0,
                                             budget, vp(FAKE), None, None, None, vp(FAKE), nb, None)

    assert call(0) == 2        # budget below 1
    assert call(129) == 2      # budget above d
    assert call(16, _prob(max_n_k=1000)) == 2   # feature-major tiles need max_n_k % 64 == 0


def test_flags_and_layout_paths(lib):
    """Unknown flag bits are rejected; problems of many shapes pass every host
    check and reach the device query (no device here: SANTA_ERR_HIP), which
    walks the workspace layout and launch-shape code paths on the host."""
    import torch
    if torch.cuda.is_available() and not os.environ.get("SANTA_ABI_SANITIZED"):
        pytest.skip("would launch kernels on fake pointers on a GPU machine")
    vp = ctypes.c_void_p
    p = _prob(flags=4)
    assert _decode(lib, p) == 3
    for B, Hq, Hkv, d, n in ((1, 32, 8, 128, 32768), (16, 32, 8, 128, 32768), (3, 8, 4, 64, 777),
                             (70, 1, 1, 64, 32768), (1, 4, 1, 64, 300123)):
        for flags in (0, santa.DETERMINISTIC):
            pr = _prob(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, max_n_k=n, flags=flags)
            nb = santa.workspace_bytes(pr)
            assert nb > 0 and nb % 256 == 0
            for mode in (0, 1, 2):
                assert _decode(lib, pr, S=64, mode=mode, ws_bytes=nb) == 6
            assert lib.santa_dense_decode(ctypes.byref(pr), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                          vp(FAKE), nb, None) == 6
    assert lib.santa_stream_read(None, 16, 1, vp(FAKE), None) == 1
    assert lib.santa_stream_read(vp(FAKE), 15, 1, vp(FAKE), None) == 2
    assert lib.santa_stream_read(vp(FAKE), 16, 9, vp(FAKE), None) == 2
