"""Pins for the oracle's Philox4x32-10 and its uniform stream layout (CPU)."""

import os

import numpy as np

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals = [int(x, 16) for x in line.split()]
            assert len(vals) == 10
            rows.append((vals[0:4], vals[4:6], vals[6:10]))
    return rows


def test_known_answer_vectors():
    rows = _kat_rows()
    assert len(rows) == 3
    for ctr, key, expect in rows:
        got = philox.philox4x32_10(*ctr, *key)
        assert [int(x) for x in got] == expect


def test_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2**32, size=(50, 4), dtype=np.uint64)
    key = rng.integers(0, 2**32, size=(50, 2), dtype=np.uint64)
    vec = philox.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], key[:, 0], key[:, 1])
    for i in range(50):
        one = philox.philox4x32_10(*[int(c) for c in ctr[i]], int(key[i, 0]), int(key[i, 1]))
        assert [int(v[i]) for v in vec] == [int(x) for x in one]


def test_stream_layout_word_k_of_block_k_over_4():
    seed = 0x0123456789ABCDEF
    row, tag = 77, philox.TAG_STRATIFIED
    words = philox.stream_words(seed, row, tag, 11)
    for k in range(11):
        block = philox.philox4x32_10(k >> 2, row, tag, 0, seed & 0xFFFFFFFF, seed >> 32)
        assert int(words[k]) == int(block[k & 3])


def test_stream_rows_broadcast():
    rows = np.arange(6)
    w = philox.stream_words(9, rows, philox.TAG_IID, 7)
    assert w.shape == (6, 7)
    for r in rows:
        assert np.array_equal(w[r], philox.stream_words(9, int(r), philox.TAG_IID, 7))


def test_uniform_conversion_is_exact_dyadic():
    words = np.array([0, 255, 256, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    u = philox.words_to_uniform(words)
    assert u[0] == 0.0 and u[1] == 0.0
    assert u[2] == 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24
    assert u[4] == 0.5
    # every value is representable in fp32 without rounding
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)


def test_uniforms_are_roughly_uniform():
    u = philox.uniforms(3, np.arange(64), philox.TAG_IID, 1024).ravel()
    assert u.min() >= 0.0 and u.max() < 1.0
    hist, _ = np.histogram(u, bins=16, range=(0.0, 1.0))
    expected = u.size / 16
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 45.0  # 15 dof; p ~ 1e-4


def test_distinct_tags_and_seeds_give_distinct_streams():
    a = philox.stream_words(1, 0, philox.TAG_SYSTEMATIC, 8)
    b = philox.stream_words(1, 0, philox.TAG_STRATIFIED, 8)
    c = philox.stream_words(2, 0, philox.TAG_SYSTEMATIC, 8)
    d = philox.stream_words(1 << 32, 0, philox.TAG_SYSTEMATIC, 8)
    assert not np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert not np.array_equal(a, d)
