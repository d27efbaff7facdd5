"""Comparison helpers for GPU-vs-oracle parity tests.

Index parity rule (``oracle/parity.py``): the sampled index of point k must
equal the oracle's, except when the point lies within `band` of every CDF value
separating the two indices (the GPU accumulates the CDF from fp32 scores, the
oracle in fp64 from exact inputs, so a point that close to a boundary may fall
on either side).  Such excused flips are counted and reported.
"""

import numpy as np
import torch

from oracle import parity as OP
from oracle import santa as O

BAND = 1e-5          # excused distance for GPU vs oracle (fp64 scores)
BAND_SAME_SCORES = 1e-6  # excused distance when the oracle reuses the GPU's scores
OUT_TOL = 2e-3       # max-abs error of the SANTA output
DENSE_TOL = 1e-3     # max-abs error of the dense output


IndexReport = OP.IndexReport
compare_indices = OP.compare_indices
compare_head = OP.compare_head
min_boundary_distance = OP.min_boundary_distance


def oracle_estimate_from_indices(V, idx, n_k, Hq, S):
    """(1/S) sum_k V[i_k] in fp64 for a GPU index list (B, H_q, S)."""
    B, Hkv = V.shape[0], V.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, V.shape[3]), np.nan)
    for b in range(B):
        if not 1 <= int(n_k[b]) <= V.shape[2]:
            continue
        for h in range(Hq):
            out[b, h] = O.gather_average(V[b, h // G].astype(np.float64), idx[b, h], S)
    return out


def to_dev(wl, device="cuda"):
    return (torch.from_numpy(wl.q).to(device), torch.from_numpy(wl.K).to(device),
            torch.from_numpy(wl.V).to(device), torch.from_numpy(wl.n_k.astype(np.int32)).to(device))
