"""Pins for the oracle's OCP E4M3 decoding and the fp8-key decode driver (CPU)."""

import numpy as np
import torch

from oracle import fp8, santa
from stochastic_sparse_decode_amd import workloads as W


def test_e4m3_table_matches_torch_float8_e4m3fn():
    # a library routine: torch's float8_e4m3fn is the same OCP E4M3 encoding
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.E4M3_TABLE
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert np.array_equal(np.signbit(got[m]), np.signbit(ref[m]))  # signed zeros too


def test_e4m3_closed_forms():
    v = fp8.E4M3_TABLE
    assert v[0x00] == 0.0 and np.signbit(v[0x80]) and v[0x80] == 0.0
    assert v[0x01] == 2.0 ** -9                 # smallest subnormal
    assert v[0x07] == 7.0 / 8.0 * 2.0 ** -6     # largest subnormal
    assert v[0x08] == 2.0 ** -6                 # smallest normal
    assert v[0x38] == 1.0 and v[0xB8] == -1.0   # E = 7 is the bias
    assert v[0x3C] == 1.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2               # no infinities, two NaN codes
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)             # codes 0..0x7E increase strictly
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])


def test_quantized_cache_rounds_to_nearest_code():
    wl = W.random_case(2, 4, 2, 64, [300, 257], seed=5)
    K8, ks = W.quantize_keys_fp8(wl.K, wl.n_k)
    finite = fp8.E4M3_TABLE[:0x7F]
    for b in range(2):
        n = int(wl.n_k[b])
        x = wl.K[b, :, :n].astype(np.float32) / ks[b][:, None, None]
        got = fp8.decode(K8[b, :, :n])
        # no representable value is strictly closer than the chosen one
        d_best = np.min(np.abs(np.abs(x)[..., None] - finite), axis=-1)
        assert np.allclose(np.abs(np.abs(x) - np.abs(got)), d_best, rtol=0, atol=1e-12)
        assert np.abs(got).max() <= 448.0


def _fp8_case(seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, n = 2, 4, 2, 64, 200
    q = rng.standard_normal((B, Hq, d)).astype(np.float16)
    K8 = rng.integers(0, 256, size=(B, Hkv, n, d)).astype(np.uint8)
    K8[(K8 & 0x7F) == 0x7F] = 0x38  # no NaN codes
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float16)
    return q, K8, V, np.array([n, 150], dtype=np.int32)


def test_fp8_keys_reduce_to_the_fp16_path_on_decoded_values():
    # every E4M3 value is exact in fp16, so with k_scale = 1 the fp8 step is
    # the plain step on the decoded keys, given as an fp16 array
    q, K8, V, n_k = _fp8_case(1)
    K16 = fp8.decode(K8).astype(np.float16)
    assert np.array_equal(K16.astype(np.float64), fp8.decode(K8))
    ones = np.ones(K8.shape[:2], dtype=np.float32)
    for mode in (0, 1, 2):
        o1, i1 = santa.santa_decode_fp8k(q, K8, ones, V, n_k, 16, mode, 3, 0.125)
        o2, i2 = santa.santa_decode(q, K16, V, n_k, 16, mode, 3, 0.125)
        assert np.array_equal(i1, i2)
        assert np.allclose(o1, o2, rtol=0, atol=1e-15)


def test_fp8_key_scale_multiplies_the_scores():
    # a power-of-two scale per KV head is exact: same result as folding it
    # into the softmax scale of a single-KV-head problem
    q, K8, V, n_k = _fp8_case(2)
    ks = np.array([[0.25, 4.0], [2.0, 0.5]], dtype=np.float32)
    s = santa.all_scores(q, fp8.dequantize(K8, ks), n_k, 0.125)
    s1 = santa.all_scores(q, fp8.decode(K8), n_k, 0.125)
    G = q.shape[1] // K8.shape[1]
    for b in range(2):
        for h in range(q.shape[1]):
            m = ~np.isnan(s1[b, h])
            assert np.array_equal(s[b, h, m], s1[b, h, m] * float(ks[b, h // G]))
