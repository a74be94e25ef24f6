"""Pins for the oracle's dispatch (nvfp4moe README, "Grouped GEMM" and "Training").

The oracle places (t, j) with a counting sort.  These tests check it against
an independent characterisation of the same permutation -- the row of (t, j)
is the number of entries with a smaller expert id plus the number of entries
with the same id and a smaller token index -- by brute force over every
routing of a tiny layer, and against the invariants the pages state
(m_indptr of length E+1, empty experts valid, counts summing to T*k).
"""
import itertools

import numpy as np
import pytest

from mixture_experts_routed_dispatch_amd import inputs


def rank_definition(ids):
    """Row of each (t, j) from its definition as a rank, O((T k)^2)."""
    T, k = ids.shape
    flat = [(int(ids[t, j]), t, j) for t in range(T) for j in range(k)]
    slots = np.zeros((T, k), np.int32)
    for (e, t, j) in flat:
        slots[t, j] = sum(1 for (e2, t2, _) in flat if e2 < e or (e2 == e and t2 < t))
    return slots


def check_invariants(ids, scores, E, m_indptr, gather, slots, probs):
    T, k = ids.shape
    R = T * k
    counts = np.bincount(ids.ravel(), minlength=E)
    assert counts.sum() == R
    assert m_indptr[0] == 0 and m_indptr[E] == R
    assert np.array_equal(np.diff(m_indptr), counts)                 # width = count, empty = 0
    assert np.array_equal(np.sort(slots.ravel()), np.arange(R))     # bijection onto [0, R)
    for t in range(T):
        for j in range(k):
            r = slots[t, j]
            e = ids[t, j]
            assert gather[r] == t
            assert m_indptr[e] <= r < m_indptr[e + 1]
            assert probs[r] == scores[t, j]
    for e in range(E):                                              # ascending t inside an expert
        seg = gather[m_indptr[e]:m_indptr[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_brute_force_all_tiny_routings(orc):
    T, E, k = 3, 4, 2
    rows = [p for p in itertools.permutations(range(E), k)]        # 12 ordered distinct pairs
    scores = np.arange(T * k, dtype=np.float32).reshape(T, k) + 0.5
    n = 0
    for combo in itertools.product(rows, repeat=T):                 # 12^3 = 1728 routings
        ids = np.array(combo, np.int32)
        m_indptr, gather, slots, probs = orc.dispatch(ids, scores, E)
        assert np.array_equal(slots, rank_definition(ids))
        check_invariants(ids, scores, E, m_indptr, gather, slots, probs)
        n += 1
    assert n == 1728


@pytest.mark.parametrize("T,E,k,routing", [
    (64, 8, 2, "uniform"), (257, 16, 8, "uniform"), (300, 128, 8, "zipf"),
    (1, 128, 8, "uniform"), (33, 256, 32, "uniform"), (50, 5, 1, "uniform"),
])
def test_invariants_random(orc, T, E, k, routing):
    rng = np.random.default_rng(T * 1000 + E)
    ids = (inputs.uniform_routing(rng, T, E, k) if routing == "uniform"
           else inputs.zipf_routing(rng, T, E, k))
    scores = rng.random((T, k)).astype(np.float32)
    m_indptr, gather, slots, probs = orc.dispatch(ids, scores, E)
    check_invariants(ids, scores, E, m_indptr, gather, slots, probs)
    if T * k <= 400:
        assert np.array_equal(slots, rank_definition(ids))


def test_zipf_routing_has_forced_empty_experts(orc):
    rng = np.random.default_rng(0)
    ids = inputs.zipf_routing(rng, 2048, 128, 8)
    m_indptr, _, _, _ = orc.dispatch(ids, np.ones(ids.shape, np.float32), 128)
    counts = np.diff(m_indptr)
    assert (counts == 0).sum() >= 8


def test_all_tokens_on_same_experts(orc):
    T, E, k = 40, 16, 3
    ids = np.tile(np.array([5, 2, 9], np.int32), (T, 1))
    scores = np.ones((T, k), np.float32)
    m_indptr, gather, slots, probs = orc.dispatch(ids, scores, E)
    check_invariants(ids, scores, E, m_indptr, gather, slots, probs)
    assert m_indptr[2] == 0 and m_indptr[3] == T and m_indptr[5] == T and m_indptr[6] == 2 * T


def test_routing_errors(orc):
    scores = np.ones((2, 2), np.float32)
    with pytest.raises(orc.RoutingError):
        orc.dispatch(np.array([[0, 4], [1, 2]], np.int32), scores, 4)      # out of range
    with pytest.raises(orc.RoutingError):
        orc.dispatch(np.array([[0, -1], [1, 2]], np.int32), scores, 4)
    with pytest.raises(orc.RoutingError):
        orc.dispatch(np.array([[3, 3], [1, 2]], np.int32), scores, 4)      # duplicate in a row
    assert orc.check_routing(np.array([[3, 1], [1, 3]], np.int32), 4) == orc.ORC_OK
