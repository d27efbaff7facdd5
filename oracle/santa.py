"""SANTA decode-step attention, oracle side (fp64, NumPy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "Stochastic Sparse Attention for Memory-Bound Inference"
(arXiv 2605.01910), abstract.  What the abstract fixes, in this module's
words:

* plain decoding touches every key row and every value row of the cache at
  each step (first sentence);
* the method draws a small number S of key positions according to the
  softmax weights of the scores and sums only the value rows at those
  positions (second sentence);
* that average has the exact attention output as its expectation, and the
  value stage reduces to fetching rows and adding them (third sentence);
* stratified and systematic placement of the draws lower the variance
  (fourth sentence; the first arXiv version names stratified only);
* a randomised three-valued query lets the score stage skip key features
  (the sentence on Bernoulli qK^T sampling).

Where the abstract leaves a step open, the functions below take these
readings: an explicit softmax scale argument; i.i.d. draws by the inverse CDF
of sorted uniforms; equal-probability strata [k/S, (k+1)/S); weights 1/S with
duplicates counted; half-open CDF intervals (a point on F_j selects j + 1);
the CDF in key-index order; the Philox stream layout of ``philox``; keep
probability |q_i| / max|q| for the ternary queries.

Per-head functions take 1-D / 2-D float64 arrays and are written to be read
against those statements; the batched drivers only loop over (b, h).
All arithmetic is fp64 on the exactly decoded fp16 inputs.

Mode numbers: 0 = i.i.d. multinomial (inverse CDF), 1 = stratified,
2 = systematic, 3 = i.i.d. multinomial by the Gumbel-max trick.
"""

import numpy as np

from . import fp8, philox

IID = 0
STRATIFIED = 1
SYSTEMATIC = 2
GUMBEL = 3
MODES = (IID, STRATIFIED, SYSTEMATIC)
_MODE_TAG = {
    IID: philox.TAG_IID,
    STRATIFIED: philox.TAG_STRATIFIED,
    SYSTEMATIC: philox.TAG_SYSTEMATIC,
}


# ----------------------------------------------------------------------------
# per-head steps
# ----------------------------------------------------------------------------

def head_scores(q_h, K_h, scale):
    """Score stage: s_j = scale * <q, k_j> for every key j (fp64).

    The abstract's premise is that every key is read; the sampling stage needs
    the full post-softmax distribution, so every score is computed.
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    K_h = np.asarray(K_h, dtype=np.float64)
    return scale * (K_h @ q_h)


def distribution(s):
    """Post-softmax distribution over key index order.

    Returns (w, cum, F): w_j = exp(s_j - max s), cum = sequential prefix sum of
    w in key-index order, F_j = cum_j / Z with Z = cum_{n-1}, so F_{n-1} = 1
    exactly.  F is the CDF that the inverse-CDF sampler inverts.
    """
    s = np.asarray(s, dtype=np.float64)
    w = np.exp(s - np.max(s))
    cum = np.cumsum(w)  # sequential, in key order
    F = cum / cum[-1]
    return w, cum, F


def probabilities(s):
    """p_j = w_j / Z, the post-softmax distribution itself."""
    w, cum, _ = distribution(s)
    return w / cum[-1]


def points(mode, S, seed, row):
    """The S sorted points t_0 <= ... <= t_{S-1} in [0, 1) for one query head.

    * i.i.d. multinomial: S independent uniforms, sorted ascending.
    * stratified: one uniform per equal-probability stratum [k/S, (k+1)/S),
      t_k = (k + u_k) / S.
    * systematic: a single uniform offset shared by all strata,
      t_k = (k + u) / S.
    ``row`` selects the stream (b * H_q + h); uniforms come from the mode's tag.
    """
    if mode not in MODES:
        raise ValueError("unknown sampling mode %r" % (mode,))
    tag = _MODE_TAG[mode]
    k = np.arange(S, dtype=np.float64)
    if mode == SYSTEMATIC:
        u = philox.uniforms(seed, row, tag, 1)[0]
        return (k + u) / S
    u = philox.uniforms(seed, row, tag, S)
    if mode == STRATIFIED:
        return (k + u) / S
    return np.sort(u, kind="stable")


def inverse_cdf(F, t):
    """Key index of each point: the j with F_{j-1} <= t < F_j (F_{-1} = 0).

    That is the number of CDF values <= t; a point exactly on F_j goes to key
    j + 1.  The result is clamped to n - 1 (only reachable through rounding).
    """
    idx = np.searchsorted(F, t, side="right")
    return np.minimum(idx, len(F) - 1)


def gumbel_draws(s, S, seed, row):
    """i.i.d. draws by the Gumbel-max trick (the alternative to the inverse CDF
    named beside the budget variant): draw k selects
    i_k = argmax_j (s_j + g_kj), g_kj = -log(-log u_kj), with u_kj the
    open-interval uniform j of draw k of stream (seed, row, 'GUMB').  Since
    the maximum of logits perturbed by independent standard Gumbel noise falls
    on key j with probability softmax(s)_j, the S draws are i.i.d. from the
    post-softmax distribution.  A tie goes to the smaller key.

    Returns (idx (S,) in draw order, gap (S,)): gap_k is the difference
    between the winning and the second largest perturbed value of draw k (inf
    when there is one key), how close the draw came to another outcome."""
    s = np.asarray(s, dtype=np.float64)
    n = len(s)
    idx = np.zeros(S, dtype=np.int64)
    gap = np.full(S, np.inf)
    for k in range(S):
        u = philox.draw_uniforms(seed, row, philox.TAG_GUMBEL, k, n)
        v = s - np.log(-np.log(u))
        j = int(np.argmax(v))  # the first maximum: the smaller key on a tie
        idx[k] = j
        if n > 1:
            gap[k] = v[j] - np.max(np.delete(v, j))
    return idx, gap


def gather_average(V_h, idx, S):
    """The SANTA estimate: (1/S) * sum_k V[i_k], duplicates counted."""
    V_h = np.asarray(V_h, dtype=np.float64)
    return V_h[np.asarray(idx, dtype=np.int64)].sum(axis=0) / S


def dense_head(s, V_h):
    """Exact post-softmax value aggregation sum_j p_j V_j (the estimand)."""
    w, cum, _ = distribution(s)
    V_h = np.asarray(V_h, dtype=np.float64)
    return (w @ V_h) / cum[-1]


def ternary_query(q_group, u):
    """Stochastic ternary queries for the G query heads of one KV head.

    q_group: (G, d) fp64 query vectors; u: (d,) uniforms shared by the group.
    Keep probability of feature i for head h is |q_hi| / A_h with
    A_h = max_i |q_hi|; a kept feature becomes sign(q_hi) * A_h, a dropped one
    0, so E[q~] = q.  Returns (q_tilde (G, d), kept (G, d) bool, A (G,)).
    The comparison u * A < |q| is exact in fp64 (24-bit times 11-bit product).
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    A = np.max(np.abs(q_group), axis=1)
    kept = u[None, :] * A[:, None] < np.abs(q_group)
    q_tilde = np.where(kept, np.sign(q_group) * A[:, None], 0.0)
    return q_tilde, kept, A


def budget_query(q_group, u, m):
    """Budget variant of the stochastic queries, for the G heads of one KV
    head: feature i of head h is kept with probability
    pi_hi = min(1, m |q_hi| / ||q_h||_1), so about m features per head are
    kept, and a kept feature takes the value q_hi / pi_hi: q_hi itself where
    pi_hi = 1 (a clipped feature) and sign(q_hi) ||q_h||_1 / m otherwise, so
    E[q~] = q.  u (d,) uniforms (multiples of 2^-24) are shared by the group;
    q = 0 keeps nothing.

    The decision u_i < pi_hi is made exactly: with every value scaled by 2^24
    to an integer (fp16 values and the uniforms are multiples of 2^-24),
    keep <=> U_i * L1 < m * Q_hi * 2^24 and clipped <=> m * Q_hi >= L1, in
    Python integers.  Returns (q_tilde (G, d), kept (G, d) bool,
    clipped (G, d) bool, c (G,) = ||q_h||_1 / m).
    """
    q_group = np.asarray(q_group, dtype=np.float64)
    G, d = q_group.shape
    Ui = [int(round(x * 2.0 ** 24)) for x in u]
    q_tilde = np.zeros((G, d))
    kept = np.zeros((G, d), dtype=bool)
    clipped = np.zeros((G, d), dtype=bool)
    c = np.zeros(G)
    for h in range(G):
        Q = [int(round(abs(x) * 2.0 ** 24)) for x in q_group[h]]
        L1 = sum(Q)
        c[h] = L1 * 2.0 ** -24 / m
        for i in range(d):
            if Q[i] == 0:
                continue
            clipped[h, i] = m * Q[i] >= L1
            kept[h, i] = Ui[i] * L1 < m * Q[i] * 2 ** 24
            if kept[h, i]:
                q_tilde[h, i] = q_group[h, i] if clipped[h, i] else np.sign(q_group[h, i]) * c[h]
    return q_tilde, kept, clipped, c


# ----------------------------------------------------------------------------
# batched drivers
# ----------------------------------------------------------------------------

def _check_shapes(q, K, V, n_k):
    B, Hq, d = q.shape
    B2, Hkv, max_n_k, d2 = K.shape
    if B2 != B or d2 != d or V.shape != K.shape or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes q%s K%s V%s" % (q.shape, K.shape, V.shape))
    n_k = np.asarray(n_k, dtype=np.int64).reshape(-1)
    if n_k.shape != (B,):
        raise ValueError("n_k must have one entry per batch element")
    return B, Hq, Hkv, d, max_n_k, n_k


def _f64(x):
    return np.asarray(x).astype(np.float64)


def santa_decode(q, K, V, n_k, S, mode, seed, scale, score_override=None,
                 return_detail=False):
    """Oracle for one SANTA decode step.

    q: (B, H_q, d); K, V: (B, H_kv, max_n_k, d) (any float dtype, decoded to
    fp64); n_k: (B,) valid keys per sequence.  Returns (out (B, H_q, d) fp64,
    indices (B, H_q, S) int64 ascending).  A sequence with n_k outside
    [1, max_n_k] yields NaN outputs and indices -1.

    ``score_override`` (B, H_q, max_n_k), if given, replaces the score stage
    (used to re-run the later steps on externally supplied scores).
    ``return_detail`` adds a dict with per-head points and CDFs.
    """
    if S < 1:
        raise ValueError("S must be >= 1")
    if mode not in MODES + (GUMBEL,):
        raise ValueError("unknown sampling mode %r" % (mode,))
    B, Hq, Hkv, d, max_n_k, n_k = _check_shapes(q, K, V, n_k)
    G = Hq // Hkv
    qf, Kf, Vf = _f64(q), K, V
    out = np.full((B, Hq, d), np.nan)
    idx_all = np.full((B, Hq, S), -1, dtype=np.int64)
    detail = {"t": {}, "F": {}}
    for b in range(B):
        n = int(n_k[b])
        if n < 1 or n > max_n_k:
            continue
        for h in range(Hq):
            hk = h // G
            Vh = _f64(Vf[b, hk, :n])
            if score_override is None:
                s = head_scores(qf[b, h], _f64(Kf[b, hk, :n]), scale)
            else:
                s = _f64(score_override[b, h, :n])
            _, _, F = distribution(s)
            if mode == GUMBEL:
                idx, gap = gumbel_draws(s, S, seed, b * Hq + h)
                order = np.argsort(idx, kind="stable")
                idx, gap = idx[order], gap[order]
            else:
                t = points(mode, S, seed, b * Hq + h)
                idx = inverse_cdf(F, t)
            out[b, h] = gather_average(Vh, idx, S)
            idx_all[b, h] = idx
            if return_detail:
                detail["F"][(b, h)] = F
                if mode == GUMBEL:
                    detail.setdefault("gap", {})[(b, h)] = gap
                    detail.setdefault("s", {})[(b, h)] = s
                else:
                    detail["t"][(b, h)] = t
    if return_detail:
        return out, idx_all, detail
    return out, idx_all


def dense_decode(q, K, V, n_k, scale):
    """Exact attention output softmax(scale * q K^T) V per (b, h) in fp64."""
    B, Hq, Hkv, d, max_n_k, n_k = _check_shapes(q, K, V, n_k)
    G = Hq // Hkv
    qf = _f64(q)
    out = np.full((B, Hq, d), np.nan)
    for b in range(B):
        n = int(n_k[b])
        if n < 1 or n > max_n_k:
            continue
        for hk in range(Hkv):
            Kh = _f64(K[b, hk, :n])
            Vh = _f64(V[b, hk, :n])
            for g in range(G):
                h = hk * G + g
                out[b, h] = dense_head(head_scores(qf[b, h], Kh, scale), Vh)
    return out


def bernoulli_queries(q, Hkv, seed, budget=0):
    """Stochastic queries for every (b, h): (q_tilde, kept, A).

    The d uniforms of KV head (b, h_kv) come from stream row b * H_kv + h_kv of
    the 'BERN' tag and are shared by the G query heads of that KV head.
    budget = 0: ternary queries (``ternary_query``; A = max |q|); budget = m
    > 0: the budget variant (``budget_query``; A = ||q||_1 / m).
    """
    qf = _f64(q)
    B, Hq, d = qf.shape
    G = Hq // Hkv
    q_tilde = np.zeros_like(qf)
    kept = np.zeros(qf.shape, dtype=bool)
    A = np.zeros((B, Hq))
    for b in range(B):
        for hk in range(Hkv):
            u = philox.uniforms(seed, b * Hkv + hk, philox.TAG_BERNOULLI, d)
            sl = slice(hk * G, (hk + 1) * G)
            if budget > 0:
                q_tilde[b, sl], kept[b, sl], _, A[b, sl] = budget_query(qf[b, sl], u, budget)
            else:
                q_tilde[b, sl], kept[b, sl], A[b, sl] = ternary_query(qf[b, sl], u)
    return q_tilde, kept, A


def bernoulli_decode(q, K, V, n_k, S, mode, seed, scale, return_detail=False, budget=0):
    """Bernoulli qK^T mode: ternary-query scores, then the SANTA value stage.

    The scores use q~ in place of q; the softmax, points, search and estimate
    are those of ``santa_decode`` on the new scores.  Returns
    (out, indices, kept (B, H_q, d) bool) and, on request, a detail dict.
    """
    Hkv = _check_shapes(q, K, V, n_k)[2]
    q_tilde, kept, _ = bernoulli_queries(q, Hkv, seed, budget)
    res = santa_decode(q_tilde, K, V, n_k, S, mode, seed, scale,
                       return_detail=return_detail)
    if return_detail:
        out, idx, detail = res
        return out, idx, kept, detail
    out, idx = res
    return out, idx, kept


def santa_decode_fp8k(q, K8, k_scale, V, n_k, S, mode, seed, scale, score_override=None,
                      return_detail=False):
    """SANTA decode step on an fp8 key cache: the keys are
    K = k_scale[b, h_kv] * decode(K8) (OCP E4M3 bytes, decoded exactly into
    fp64 by ``fp8.dequantize``); every later step is ``santa_decode``'s."""
    K = fp8.dequantize(K8, k_scale)
    return santa_decode(q, K, V, n_k, S, mode, seed, scale, score_override=score_override,
                        return_detail=return_detail)


def gather_paged(cache, block_table, n_k, max_n_k):
    """Contiguous (B, H_kv, max_n_k, d) copy of a paged cache (same dtype).

    cache: (num_blocks, H_kv, P, d); block_table: (B, max_blocks) int; key j
    of sequence b is row j % P of block block_table[b, j // P].  Rows at and
    past n_k[b] are NaN (never read by the step).  A sequence with an invalid
    length, or whose blocks below n_k are not all in [0, num_blocks), is left
    entirely NaN.
    """
    num_blocks, Hkv, P, d = cache.shape
    B = block_table.shape[0]
    out = np.full((B, Hkv, max_n_k, d), np.nan, dtype=cache.dtype)  # exact copies of the stored values
    for b in range(B):
        n = int(n_k[b])
        if not 1 <= n <= max_n_k:
            continue
        blocks = [int(block_table[b, j]) for j in range((n + P - 1) // P)]
        if any(x < 0 or x >= num_blocks for x in blocks):
            continue
        for i, blk in enumerate(blocks):  # keys i P .. i P + rows - 1 sit in block blk
            rows = min(P, n - i * P)
            out[b, :, i * P:i * P + rows] = cache[blk, :, :rows]
    return out


def santa_decode_paged(q, K_cache, V_cache, block_table, n_k, max_n_k, S, mode, seed, scale,
                       score_override=None, return_detail=False):
    """SANTA decode step on a paged KV cache: the keys and values of every
    sequence are gathered through the block table (``gather_paged``), then
    every step is ``santa_decode``'s.  A sequence with a block-table entry out
    of range yields NaN outputs and indices -1, as an invalid length does."""
    K = gather_paged(K_cache, block_table, n_k, max_n_k)
    V = gather_paged(V_cache, block_table, n_k, max_n_k)
    n_eff = np.asarray(n_k, dtype=np.int64).copy()
    for b in range(len(n_eff)):
        if np.isnan(K[b]).all():
            n_eff[b] = 0  # invalid: NaN outputs
    return santa_decode(q, K, V, n_eff, S, mode, seed, scale, score_override=score_override,
                        return_detail=return_detail)


def all_scores(q, K, n_k, scale):
    """Scores (B, H_q, max_n_k) fp64, NaN beyond n_k (for diagnostics)."""
    qf = _f64(q)
    B, Hq, d = qf.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    max_n_k = K.shape[2]
    n_k = np.asarray(n_k, dtype=np.int64).reshape(-1)
    s = np.full((B, Hq, max_n_k), np.nan)
    for b in range(B):
        n = int(n_k[b])
        if n < 1 or n > max_n_k:
            continue
        for h in range(Hq):
            s[b, h, :n] = head_scores(qf[b, h], _f64(K[b, h // G, :n]), scale)
    return s
