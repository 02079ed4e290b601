"""Pins for oracle/segments.py: brute force with Python's sorted() and counts, and
the structural invariants of a CSR grouping (monotone offsets, last = T, permutation)."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.segments import build_segments


def _brute(ids, n):
    order = sorted(range(len(ids)), key=lambda t: (ids[t], t))
    counts = [sum(1 for i in ids if i == a) for a in range(n)]
    indptr = [0]
    for c in counts:
        indptr.append(indptr[-1] + c)
    return indptr, order


@given(st.integers(1, 40).flatmap(lambda n: st.tuples(st.just(n), st.lists(st.integers(0, n - 1), max_size=200))))
@settings(max_examples=200, deadline=None)
def test_matches_brute_force(case):
    n, ids = case
    indptr, order = build_segments(ids, n)
    bi, bo = _brute(ids, n)
    assert indptr.tolist() == bi and order.tolist() == bo


def test_invariants_and_examples():
    indptr, order = build_segments([0, 1, 1, 0], 2)
    assert indptr.tolist() == [0, 2, 4] and order.tolist() == [0, 3, 1, 2]
    indptr, order = build_segments([3, 3, 0], 5)
    assert indptr.tolist() == [0, 1, 1, 1, 3, 3] and order.tolist() == [2, 0, 1]
    indptr, order = build_segments([], 3)
    assert indptr.tolist() == [0, 0, 0, 0] and order.size == 0
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 17, 1000)
    indptr, order = build_segments(ids, 17)
    assert (np.diff(indptr) >= 0).all() and indptr[-1] == 1000
    assert sorted(order.tolist()) == list(range(1000))
    for a in range(17):
        seg = order[indptr[a]:indptr[a + 1]]
        assert (ids[seg] == a).all() and (np.diff(seg) > 0).all()


def test_rejects_bad_ids():
    with pytest.raises(ValueError):
        build_segments([0, 2], 2)
    with pytest.raises(ValueError):
        build_segments([-1], 2)
    with pytest.raises(ValueError):
        build_segments([0], 0)
