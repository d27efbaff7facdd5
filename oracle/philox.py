"""Philox4x32-10 and the sampler's uniform stream (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages name no generator; the method only needs S uniforms per query head
(systematic sampling needs one).  The counter-based Philox4x32-10 generator of
Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
(SC'11), is used because both sides can evaluate any element of the stream
independently.  This module is written from that paper's definition:

* state: four 32-bit counter words (c0, c1, c2, c3) and two key words (k0, k1);
* one round multiplies c0 by M0 and c2 by M1 as 32x32 -> 64-bit products and
  outputs (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
* between rounds the key is bumped by the Weyl constants (W0, W1);
* ten rounds.

Stream layout (a reading of this build; the pages are silent): element ``k``
of the stream identified by ``(seed, row, tag)`` is output word ``k & 3`` of
Philox4x32-10 applied to counter ``(k >> 2, row, tag, 0)`` with key
``(seed & 0xffffffff, seed >> 32)``.  A 32-bit word ``x`` becomes the uniform
``(x >> 8) * 2**-24``, an exact dyadic rational in ``[0, 1 - 2**-24]``.

The Gumbel-max sampler needs one uniform per (draw, key): element ``j`` of
draw ``k`` of stream ``(seed, row, tag)`` is output word ``j & 3`` of the
counter ``(j >> 2, row, tag, k)`` (the fourth counter word numbers the draw),
mapped into the open interval as ``((x >> 9) + 1/2) * 2**-23``: a value in
[2**-24, 1 - 2**-24] that fp32 holds exactly, so that both logarithms of the
Gumbel transform are finite on either side.

Pinned by tests/test_oracle_philox.py against the generator authors'
published known-answer vectors (tests/golden/philox4x32_10_kat.txt).
"""

import numpy as np

MASK32 = 0xFFFFFFFF
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
ROUNDS = 10

# Stream tags: the ASCII bytes of a four-letter name, one stream per use.
TAG_SYSTEMATIC = 0x53595354  # 'SYST'
TAG_STRATIFIED = 0x53545254  # 'STRT'
TAG_IID = 0x49494420  # 'IID '
TAG_BERNOULLI = 0x4245524E  # 'BERN'
TAG_GUMBEL = 0x47554D42  # 'GUMB'


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply Philox4x32-10 elementwise.

    All arguments are integers or integer arrays holding 32-bit values; they
    broadcast against each other.  Returns the four output words as uint64
    arrays holding 32-bit values.  The arithmetic is done in uint64 so that a
    32x32-bit product is exact.
    """
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    k0 = np.asarray(k0, dtype=np.uint64) & MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & MASK32
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    mask = np.uint64(MASK32)
    shift = np.uint64(32)
    for rnd in range(ROUNDS):
        if rnd > 0:
            k0 = (k0 + np.uint64(PHILOX_W0)) & mask
            k1 = (k1 + np.uint64(PHILOX_W1)) & mask
        prod0 = m0 * c0  # exact: both factors < 2**32
        prod1 = m1 * c2
        hi0, lo0 = prod0 >> shift, prod0 & mask
        hi1, lo1 = prod1 >> shift, prod1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def stream_words(seed, row, tag, count):
    """Words 0..count-1 of the stream (seed, row, tag) as uint64 (32-bit values).

    ``row`` may be an integer array; the result then has shape
    ``row.shape + (count,)``.
    """
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    k0, k1 = seed & MASK32, seed >> 32
    row = np.asarray(row, dtype=np.uint64)
    blocks = np.arange((count + 3) // 4, dtype=np.uint64)
    out = philox4x32_10(blocks, row[..., None], tag, 0, k0, k1)
    # word k sits at block k >> 2, position k & 3
    words = np.stack(out, axis=-1).reshape(row.shape + (4 * len(blocks),))
    return words[..., :count]


def words_to_uniform(words):
    """Map 32-bit words to exact dyadic uniforms (x >> 8) * 2**-24 in fp64."""
    words = np.asarray(words, dtype=np.uint64)
    return (words >> np.uint64(8)).astype(np.float64) * (2.0 ** -24)


def uniforms(seed, row, tag, count):
    """Uniforms 0..count-1 of stream (seed, row, tag), fp64 in [0, 1 - 2**-24]."""
    return words_to_uniform(stream_words(seed, row, tag, count))


def draw_uniforms(seed, row, tag, draw, count):
    """Open-interval uniforms 0..count-1 of draw ``draw`` of stream (seed, row,
    tag): word j & 3 of counter (j >> 2, row, tag, draw), as
    ((x >> 9) + 1/2) * 2**-23 in [2**-24, 1 - 2**-24], fp64 (exact)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    k0, k1 = seed & MASK32, seed >> 32
    blocks = np.arange((count + 3) // 4, dtype=np.uint64)
    out = philox4x32_10(blocks, row, tag, draw, k0, k1)
    words = np.stack(out, axis=-1).reshape(-1)[:count]
    return ((words >> np.uint64(9)).astype(np.float64) + 0.5) * (2.0 ** -23)
