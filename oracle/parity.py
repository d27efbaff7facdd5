"""Index-parity bookkeeping for comparing a sampled index list with the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): used by ``tests/`` and
by the CPU-baseline leg of ``bench.py``.

Rule (the index-parity tolerance the workload description fixes): the sampled
index of point k must equal the oracle's, except when every CDF value that
separates the two indices lies within ``band`` of the point, since a point that
close to a boundary may fall on either side when the CDF is accumulated in
another precision or order.  Such excused flips are counted and reported.
"""

from dataclasses import dataclass

import numpy as np


@dataclass
class IndexReport:
    points: int = 0
    exact: int = 0
    excused: int = 0
    bad: int = 0
    heads_with_flips: int = 0

    def add(self, other):
        for f in ("points", "exact", "excused", "bad", "heads_with_flips"):
            setattr(self, f, getattr(self, f) + getattr(other, f))
        return self

    def as_dict(self):
        return {"points": self.points, "exact": self.exact, "excused": self.excused, "bad": self.bad,
                "heads_with_flips": self.heads_with_flips}

    def __str__(self):
        return ("points=%d exact=%d excused(<band)=%d bad=%d heads_with_flips=%d"
                % (self.points, self.exact, self.excused, self.bad, self.heads_with_flips))


def compare_head(idx_gpu, idx_or, t, F, band):
    """Compare one head's index lists (S,) given the oracle's points t and CDF F."""
    rep = IndexReport(points=len(idx_or))
    diff = np.nonzero(np.asarray(idx_gpu) != np.asarray(idx_or))[0]
    rep.exact = len(idx_or) - len(diff)
    rep.heads_with_flips = 1 if len(diff) else 0
    for k in diff:
        lo, hi = sorted((int(idx_gpu[k]), int(idx_or[k])))
        if lo < 0 or hi >= len(F):
            rep.bad += 1
            continue
        between = F[lo:hi]  # CDF values separating the two keys
        if len(between) and np.all(np.abs(between - t[k]) < band):
            rep.excused += 1
        else:
            rep.bad += 1
    return rep


def compare_indices(idx_gpu, idx_or, detail, band, flips_out=None):
    """Compare (B, H, S) index arrays using the oracle's points and CDFs
    (``detail`` as returned by the oracle's decode with return_detail=True)."""
    rep = IndexReport()
    B, H, S = idx_or.shape
    for b in range(B):
        for h in range(H):
            if (b, h) not in detail["t"]:
                continue  # invalid sequence
            sub = compare_head(idx_gpu[b, h], idx_or[b, h], detail["t"][(b, h)], detail["F"][(b, h)], band)
            if sub.heads_with_flips and flips_out is not None:
                flips_out.add((b, h))
            rep.add(sub)
    return rep


def min_boundary_distance(t, F):
    """Smallest distance between any point of t and any CDF value of F."""
    t = np.asarray(t, dtype=np.float64)
    i = np.searchsorted(F, t)
    below = np.where(i > 0, np.abs(t - F[np.maximum(i - 1, 0)]), np.inf)
    above = np.where(i < len(F), np.abs(F[np.minimum(i, len(F) - 1)] - t), np.inf)
    return float(min(below.min(), above.min()))
