"""moe_replan (host C++ in libmoe_arena) against the oracle's re-plan.

moe_replan makes no HIP call, so these run on the CPU: bit-exact evict/load
lists and slot tables on random tables with heavy ties, the 40-layer arena's
real shape (6666 slots, 333 swaps), floors, degenerate cases and rejects.
"""
import ctypes

import numpy as np
import pytest

import fixtures
from oracle import plan
from resident_expert_routing_amd import binding as B


def lib_replan(hist, es, k, n_swap):
    L, E = es.shape
    hist = np.ascontiguousarray(hist, dtype=np.float64)
    es32 = np.ascontiguousarray(es, dtype=np.int32)
    ev = np.full((max(n_swap, 1), 2), -7, dtype=np.int32)
    ld = np.full((max(n_swap, 1), 2), -7, dtype=np.int32)
    new = np.empty_like(es32)
    n = ctypes.c_int(-1)
    st = B.moe_replan(hist, es32, L, E, k, n_swap, ev, ld, new, n)
    B.check(st, "moe_replan")
    nd = n.value
    return [tuple(map(int, p)) for p in ev[:nd]], [tuple(map(int, p)) for p in ld[:nd]], new


def oracle_replan(hist, es, k, n_swap):
    ev, ld, new = plan.replan(hist, es, n_swap, k)
    m = min(len(ev), len(ld))      # the oracle pairs the i-th eviction with the i-th load
    return [tuple(map(int, p)) for p in ev[:m]], [tuple(map(int, p)) for p in ld[:m]], new


def random_table(rng, L, E, lo, hi):
    es = np.full((L, E), -1, dtype=np.int32)
    nxt = 0
    for l in range(L):
        c = int(rng.integers(lo, hi + 1))
        es[l, rng.choice(E, c, replace=False)] = np.arange(nxt, nxt + c)
        nxt += c
    perm = rng.permutation(nxt)          # slots scattered over layers
    es[es >= 0] = perm[es[es >= 0]]
    return es


def test_replan_matches_oracle_random_with_ties():
    rng = np.random.default_rng(21)
    for trial in range(200):
        L, E = int(rng.integers(1, 7)), int(rng.integers(2, 40))
        k = int(rng.integers(1, min(E, 8) + 1))
        es = random_table(rng, L, E, 0, E)
        hist = rng.integers(0, 5, size=(L, E)).astype(np.float64)
        if trial % 3 == 0:
            hist = rng.random((L, E))
        if trial % 7 == 0:
            hist[hist == 0] = -0.0           # -0 ties with +0
        n_swap = int(rng.integers(0, L * E + 2))
        got = lib_replan(hist, es, k, n_swap)
        want = oracle_replan(hist, es, k, n_swap)
        assert got[0] == want[0] and got[1] == want[1], trial
        assert np.array_equal(got[2], want[2]), trial


def test_replan_arena40_shape():
    """The 40-layer arena: 6666 slots, 333 swaps, per-layer floor k = 8."""
    counts = fixtures.arena40_layer_counts()
    assert counts.sum() == 6666
    rng = np.random.default_rng(22)
    L, E, k = 40, 256, 8
    es = np.full((L, E), -1, dtype=np.int32)
    nxt = 0
    for l in range(L):
        es[l, rng.choice(E, int(counts[l]), replace=False)] = np.arange(nxt, nxt + counts[l])
        nxt += int(counts[l])
    # demand shaped like a Zipf router: a few hot experts per layer, most cold, many zeros
    hist = np.where(rng.random((L, E)) < 0.3, 0.0, rng.pareto(1.2, (L, E)) * 3)
    n_swap = 6666 // 20
    got = lib_replan(hist, es, k, n_swap)
    want = oracle_replan(hist, es, k, n_swap)
    assert len(got[0]) == 333
    assert got[0] == want[0] and got[1] == want[1]
    assert np.array_equal(got[2], want[2])
    new = got[2]
    assert sorted(new[new >= 0]) == list(range(6666))          # every slot still used once
    assert ((new >= 0).sum(axis=1) >= np.minimum((es >= 0).sum(axis=1), k)).all()


def test_replan_floor_blocks_every_eviction():
    es = np.array([[0, 1, -1, -1], [2, 3, -1, -1]], dtype=np.int32)
    hist = np.array([[0.0, 0.0, 9.0, 9.0], [0.0, 0.0, 9.0, 9.0]])
    ev, ld, new = lib_replan(hist, es, k=2, n_swap=3)
    assert ev == [] and ld == [] and np.array_equal(new, es)


def test_replan_fewer_candidates_than_swaps():
    es = np.array([[0, 1, 2, -1]], dtype=np.int32)
    hist = np.array([[1.0, 2.0, 3.0, 0.5]])
    ev, ld, new = lib_replan(hist, es, k=1, n_swap=3)
    # two evictable, one non-resident: one swap, even though it moves a colder expert in
    assert ev == [(0, 0)] and ld == [(0, 3)]
    assert new.tolist() == [[-1, 1, 2, 0]]
    assert oracle_replan(hist, es, 1, 3)[0] == ev


def test_replan_zero_swaps():
    es = np.array([[0, -1], [-1, 1]], dtype=np.int32)
    ev, ld, new = lib_replan(np.ones((2, 2)), es, k=1, n_swap=0)
    assert ev == [] and np.array_equal(new, es)


def test_replan_rejects():
    es = np.array([[0, 1, -1]], dtype=np.int32)
    h = np.zeros((1, 3))
    ev = np.zeros((2, 2), np.int32)
    ld = np.zeros((2, 2), np.int32)
    new = np.zeros_like(es)
    n = ctypes.c_int()
    r = B.moe_replan
    assert r(None, es, 1, 3, 1, 2, ev, ld, new, n) == B.MOE_EINVAL
    assert r(h, es, 0, 3, 1, 2, ev, ld, new, n) == B.MOE_EINVAL
    assert r(h, es, 1, 3, 0, 2, ev, ld, new, n) == B.MOE_EINVAL
    assert r(h, es, 1, 3, 1, -1, ev, ld, new, n) == B.MOE_EINVAL
    assert r(h, es, 1, 3, 1, 2, None, ld, new, n) == B.MOE_EINVAL
    assert r(h, es, 1, 3, 40, 2, ev, ld, new, n) == B.MOE_EUNSUPPORTED
    hn = h.copy()
    hn[0, 2] = np.nan
    assert r(hn, es, 1, 3, 1, 2, ev, ld, new, n) == B.MOE_EINVAL
    dup = np.array([[0, 0, -1]], dtype=np.int32)
    assert r(h, dup, 1, 3, 1, 2, ev, ld, new, n) == B.MOE_EINVAL
