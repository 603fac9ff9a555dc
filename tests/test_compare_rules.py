"""Host checks of the acceptance comparison rule: only the decision at which
two walks part may excuse a difference, and only when it is a near tie."""
import numpy as np
import pytest

import oracle
from tests.devutil import compare_accept, decisive_events


def _case(u_children, u_root=0.0):
    """Root with three children (tokens 3, 5, 1); p = 1/8, q = 1/4 (so a
    child is accepted iff u < 1/2); leaves draw with u = 0."""
    V, n = 8, 3
    parent = np.array([[-1, 0, 0, 0]], np.int32)
    tok = np.array([[0, 3, 5, 1]], np.int32)
    logits = np.zeros((1, n + 1, V), np.float32)
    qd = np.full((1, n + 1, V), 0.25, np.float32)
    unif = np.zeros((1, n + 1, 2), np.float32)
    unif[0, 1:, 0] = u_children
    unif[0, 0, 1] = u_root
    return oracle.accept(logits, "f32", qd, parent, tok, unif, 1.0, trace=True)


def test_decisive_event_is_the_smaller_diverging_child():
    path, plen, bonus, ev = _case([0.7, 0.5, 0.2])   # oracle: rejects 1, 2 (u = 0.5 is not < 0.5), takes 3
    assert list(path[0, :plen[0]]) == [0, 3]
    gpu_row = np.array([0, 2, -1, -1])               # a walk that accepted child 2 instead
    dec = decisive_events(gpu_row, 2, path[0], int(plen[0]), ev[0])
    assert len(dec) == 1 and dec[0][0] == "test" and dec[0][2] == 2
    # child 2's test sits exactly on the boundary (r/q = 1/2 = u): excused
    assert compare_accept((gpu_row[None], np.array([2]), bonus), (path, plen, bonus), ev) == 1


def test_difference_away_from_the_decisive_event_is_not_excused():
    path, plen, bonus, ev = _case([0.5, 0.9, 0.2])   # child 1 is the near tie; oracle takes 3
    assert list(path[0, :plen[0]]) == [0, 3]
    gpu_row = np.array([0, 2, -1, -1])               # parts at child 2, which is not a near tie
    with pytest.raises(AssertionError):
        compare_accept((gpu_row[None], np.array([2]), bonus), (path, plen, bonus), ev)


def test_bonus_difference_needs_a_near_tie_sample():
    path, plen, bonus, ev = _case([0.9, 0.9, 0.9], u_root=0.5)   # all rejected; bonus = invcdf(p, 0.5) = 4
    assert plen[0] == 1 and bonus[0] == 4
    # u * Z = 0.5 sits on the CDF boundary between tokens 3 and 4: 3 is excused
    assert compare_accept((path, plen, np.array([3])), (path, plen, bonus), ev) == 1
    with pytest.raises(AssertionError):
        compare_accept((path, plen, np.array([6])), (path, plen, bonus), ev)
