"""Seeded synthetic inputs for SANTA decode steps.

This module only draws inputs: it holds none of the method's arithmetic
(no scores, no softmax, no sampling).  The tests, the benchmark and the
oracle-side checks all take their inputs from here, so that the oracle and the
GPU path see the same bytes.

Recipe (every config is generated from ``numpy.random.default_rng(seed)``,
normal draws in float32, rounded to fp16 with round-to-nearest-even):

* ``tiny``     1 query head, 1 KV head, d=64, n_k=1024; K, V ~ N(0, 1);
               q ~ N(0, 1)/sqrt(d) with the softmax scale folded in (scale=1);
               4 keys at distinct random positions set to 3 q/|q|.
* ``llama``    Llama-3.1-8B attention shape: 32 query heads, 8 KV heads,
               d=128, scale 1/sqrt(d); q, K, V ~ N(0, 1); 1% of the keys of
               each (sequence, KV head) are heavy hitters aligned with the
               normalised sum g of the group's query vectors: position 0 (the
               attention sink) holds 2 sqrt(d) g, ceil(0.01 n_k) - 1 further
               distinct random positions hold sqrt(d) g.  V is not planted.
               Batched variants draw n_k per sequence uniformly in a range and
               pad every sequence to max_n_k rows.
* ``sweep``    no planting; q = r sqrt(d) z/|z| with z ~ N(0, I), so the
               logit standard deviation is r (near-uniform to peaked).
* ``bernoulli`` q, K, V ~ N(0, 1), no planting.

Rows beyond a sequence's n_k are filled with ``pad_value`` (NaN by default in
tests, so that any read of padding poisons the result).
"""

from dataclasses import dataclass, field

import numpy as np

FP16 = np.float16


@dataclass
class Workload:
    name: str
    q: np.ndarray  # (B, H_q, d) fp16
    K: np.ndarray  # (B, H_kv, max_n_k, d) fp16
    V: np.ndarray  # (B, H_kv, max_n_k, d) fp16
    n_k: np.ndarray  # (B,) int32
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.K.shape[1]

    @property
    def d(self):
        return self.q.shape[2]

    @property
    def max_n_k(self):
        return self.K.shape[2]


def _normal16(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32).astype(FP16)


def _pad(x, n_k, pad_value):
    if pad_value is None:
        return
    for b, n in enumerate(n_k):
        x[b, :, int(n):, :] = pad_value


def plant_heavy_hitters(rng, q, K, n_k, frac=0.01, sink=True):
    """Overwrite 1% of each (b, h_kv) key block with keys aligned to the group.

    The direction g is the normalised sum of the group's (fp16-decoded) query
    vectors; planted keys are sqrt(d) g, and the sink at index 0 is 2 sqrt(d) g.
    """
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    planted = {}
    for b in range(B):
        n = int(n_k[b])
        for hk in range(Hkv):
            g = q[b, hk * G:(hk + 1) * G].astype(np.float64).sum(axis=0)
            norm = np.linalg.norm(g)
            g = g / norm if norm > 0 else g
            P = int(np.ceil(frac * n))
            others = rng.choice(np.arange(1, n), size=max(P - 1, 0), replace=False) if n > 1 else []
            pos = np.concatenate(([0], np.sort(np.asarray(others, dtype=np.int64))))
            K[b, hk, pos] = (np.sqrt(d) * g).astype(FP16)
            if sink:
                K[b, hk, 0] = (2.0 * np.sqrt(d) * g).astype(FP16)
            planted[(b, hk)] = pos
    return planted


def tiny(seed=1000, n_k=1024, d=64, n_planted=4):
    """Single-head case: 1 query, 1 KV head, d=64, n_k=1024, 4 planted keys."""
    rng = np.random.default_rng(seed)
    K = _normal16(rng, (1, 1, n_k, d))
    V = _normal16(rng, (1, 1, n_k, d))
    q = (rng.standard_normal(size=(1, 1, d)) / np.sqrt(d)).astype(FP16)
    qd = q[0, 0].astype(np.float64)
    pos = rng.choice(n_k, size=n_planted, replace=False)
    K[0, 0, pos] = (3.0 * qd / np.linalg.norm(qd)).astype(FP16)
    return Workload("tiny", q, K, V, np.array([n_k], dtype=np.int32), 1.0,
                    {"planted": np.sort(pos), "seed": seed})


def random_case(B, Hq, Hkv, d, n_k, max_n_k=None, seed=0, planted=False,
                q_scale=1.0, scale=None, pad_value=None):
    """General case used by tests: any shape, ragged n_k, optional planting."""
    rng = np.random.default_rng(seed)
    n_k = np.broadcast_to(np.asarray(n_k, dtype=np.int32), (B,)).copy()
    if max_n_k is None:
        max_n_k = int(n_k.max())
    q = (q_scale * rng.standard_normal(size=(B, Hq, d), dtype=np.float32)).astype(FP16)
    K = _normal16(rng, (B, Hkv, max_n_k, d))
    V = _normal16(rng, (B, Hkv, max_n_k, d))
    meta = {"seed": seed}
    if planted:
        meta["planted"] = plant_heavy_hitters(rng, q, K, np.minimum(n_k, max_n_k))
    _pad(K, np.clip(n_k, 0, max_n_k), pad_value)
    _pad(V, np.clip(n_k, 0, max_n_k), pad_value)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return Workload("random", q, K, V, n_k, float(scale), meta)


def llama(B=1, n_k=32768, seed=1001, n_k_range=None, max_n_k=None,
          pad_value=None, Hq=32, Hkv=8, d=128, planted=True):
    """Llama-3.1-8B-shaped decode layer (32/8 heads, d=128) with heavy hitters.

    ``n_k_range=(lo, hi)`` draws each sequence's n_k uniformly in [lo, hi]
    (batched long-context case); buffers are padded to ``max_n_k``.
    """
    rng = np.random.default_rng(seed)
    if n_k_range is not None:
        lo, hi = n_k_range
        nk = rng.integers(lo, hi + 1, size=B).astype(np.int32)
        max_n_k = max_n_k or hi
    else:
        nk = np.full(B, n_k, dtype=np.int32)
        max_n_k = max_n_k or n_k
    q = _normal16(rng, (B, Hq, d))
    K = _normal16(rng, (B, Hkv, max_n_k, d))
    V = _normal16(rng, (B, Hkv, max_n_k, d))
    meta = {"seed": seed}
    if planted:
        meta["planted"] = plant_heavy_hitters(rng, q, K, nk)
    _pad(K, nk, pad_value)
    _pad(V, nk, pad_value)
    return Workload("llama", q, K, V, nk, 1.0 / np.sqrt(d), meta)


def sweep(B=4, n_k=4096, r=1.0, seed=1003, Hq=32, Hkv=8, d=128):
    """Context sweep: unplanted K, V; query norm r sqrt(d) sets the logit spread."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(size=(B, Hq, d))
    q = (r * np.sqrt(d) * z / np.linalg.norm(z, axis=-1, keepdims=True)).astype(FP16)
    K = _normal16(rng, (B, Hkv, n_k, d))
    V = _normal16(rng, (B, Hkv, n_k, d))
    nk = np.full(B, n_k, dtype=np.int32)
    return Workload("sweep", q, K, V, nk, 1.0 / np.sqrt(d), {"seed": seed, "r": r})


def bernoulli(B=8, n_k=32768, seed=1004, Hq=32, Hkv=8, d=128):
    """Bernoulli qK^T case: q, K, V ~ N(0, 1), no planting."""
    rng = np.random.default_rng(seed)
    q = _normal16(rng, (B, Hq, d))
    K = _normal16(rng, (B, Hkv, n_k, d))
    V = _normal16(rng, (B, Hkv, n_k, d))
    nk = np.full(B, n_k, dtype=np.int32)
    return Workload("bernoulli", q, K, V, nk, 1.0 / np.sqrt(d), {"seed": seed})


def feature_major(K, tile=64):
    """Relayout K (B, H_kv, n, d) into 64-key feature-major tiles (B, H_kv, n/64, d, 64).

    A layout change only (used to build expected bytes for the packing kernel).
    """
    B, Hkv, n, d = K.shape
    if n % tile:
        raise ValueError("max_n_k must be a multiple of %d" % tile)
    return np.ascontiguousarray(K.reshape(B, Hkv, n // tile, tile, d).transpose(0, 1, 2, 4, 3))


def quantize_keys_fp8(K, n_k):
    """fp8 key cache for K (B, H_kv, max_n_k, d) fp16: (K8 uint8, k_scale).

    One fp32 scale per (sequence, KV head), k_scale = max |K| / 448 over the
    sequence's valid rows (1 when that maximum is 0 or the length is invalid),
    and K8 = the OCP E4M3 bytes of K / k_scale, rounded to nearest even (by
    torch's float8_e4m3fn conversion); so the cache holds
    K ~ k_scale * decode(K8).  Rows past n_k keep whatever K / k_scale gives
    (NaN padding stays NaN).  This is input preparation, as when a serving
    system writes its cache; the decode step only reads K8 and k_scale.
    """
    import torch

    B, Hkv, max_n_k, d = K.shape
    k_scale = np.ones((B, Hkv), dtype=np.float32)
    for b in range(B):
        n = int(n_k[b])
        if not 1 <= n <= max_n_k:
            continue
        amax = np.abs(K[b, :, :n].astype(np.float32)).max(axis=(1, 2))
        k_scale[b] = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    x = torch.from_numpy(K.astype(np.float32) / k_scale[:, :, None, None])
    K8 = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return K8, k_scale


def paginate(K, V, n_k, block_size, seed=0, spare_blocks=3):
    """Paged copy of a contiguous cache: (K_cache, V_cache, block_table, num_blocks).

    Each sequence's rows below n_k are cut into blocks of ``block_size`` keys;
    the blocks are placed at shuffled positions of a pool of num_blocks =
    (blocks used) + spare_blocks; the rows of a last, partly used block past
    n_k and the spare blocks are NaN (a read of them poisons the result).  K_cache, V_cache: (num_blocks, H_kv, block_size,
    d) fp16; block_table: (B, max_blocks) int32, entries past a sequence's
    blocks set to -1.  Sequences with an invalid n_k get no blocks.
    """
    B, Hkv, max_n_k, d = K.shape
    P = int(block_size)
    max_blocks = (max_n_k + P - 1) // P
    rng = np.random.default_rng(seed)
    owners = []
    for b in range(B):
        n = int(n_k[b])
        if 1 <= n <= max_n_k:
            owners += [(b, i) for i in range((n + P - 1) // P)]
    num_blocks = len(owners) + spare_blocks
    place = rng.permutation(num_blocks)[:len(owners)]
    Kc = np.full((num_blocks, Hkv, P, d), np.nan, dtype=FP16)
    Vc = np.full((num_blocks, Hkv, P, d), np.nan, dtype=FP16)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    for (b, i), pos in zip(owners, place):
        n = int(n_k[b])
        rows = min(P, n - i * P)
        Kc[pos, :, :rows] = K[b, :, i * P:i * P + rows]
        Vc[pos, :, :rows] = V[b, :, i * P:i * P + rows]
        table[b, i] = pos
    return Kc, Vc, table, num_blocks
