"""Pins for the index-parity bookkeeping (oracle/parity.py), on hand-made CDFs."""

import numpy as np

from oracle import parity as OP


def test_flip_across_a_near_boundary_is_excused_and_a_far_one_is_bad():
    F = np.array([0.1, 0.25, 0.5, 0.75, 1.0])
    t = np.array([0.05, 0.25 - 3e-6, 0.6, 0.9])
    ref = np.searchsorted(F, t, side="right")  # [0, 1, 3, 4]
    assert list(ref) == [0, 1, 3, 4]
    got = ref.copy()
    got[1] = 2        # across F[1] = 0.25, 3e-6 away: excused at band 1e-5, not at 1e-6
    got[2] = 1        # across F[1] and F[2], 0.1 away: bad
    rep = OP.compare_head(got, ref, t, F, 1e-5)
    assert (rep.points, rep.exact, rep.excused, rep.bad, rep.heads_with_flips) == (4, 2, 1, 1, 1)
    rep = OP.compare_head(got, ref, t, F, 1e-6)
    assert (rep.excused, rep.bad) == (0, 2)


def test_out_of_range_index_is_bad_and_equal_lists_are_exact():
    F = np.linspace(0.1, 1.0, 10)
    t = np.array([0.15, 0.55])
    ref = np.searchsorted(F, t, side="right")
    assert OP.compare_head(ref, ref, t, F, 1e-5).as_dict() == dict(points=2, exact=2, excused=0, bad=0,
                                                                   heads_with_flips=0)
    assert OP.compare_head(np.array([-1, ref[1]]), ref, t, F, 1.0).bad == 1
    assert OP.compare_head(np.array([ref[0], 10]), ref, t, F, 1.0).bad == 1


def test_compare_indices_skips_invalid_sequences_and_collects_flipped_heads():
    F = np.array([0.5, 1.0])
    det = {"t": {(0, 0): np.array([0.25, 0.75]), (0, 1): np.array([0.5 - 1e-7, 0.9])}, "F": {(0, 0): F, (0, 1): F}}
    ref = np.array([[[0, 1], [0, 1], [-1, -1]]])  # head 2: invalid, not in the detail
    got = ref.copy()
    got[0, 1, 0] = 1
    flips = set()
    rep = OP.compare_indices(got, ref, det, 1e-5, flips)
    assert (rep.points, rep.exact, rep.excused, rep.bad) == (4, 3, 1, 0) and flips == {(0, 1)}


def test_min_boundary_distance():
    F = np.array([0.2, 0.5, 1.0])
    assert abs(OP.min_boundary_distance([0.3, 0.49], F) - 0.01) < 1e-15
    assert OP.min_boundary_distance([0.5], F) == 0.0
    assert abs(OP.min_boundary_distance([0.05], F) - 0.15) < 1e-15
