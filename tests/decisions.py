"""Comparing a GPU decision (hot read, re-plan, ring plan) with the oracle's.

The oracle takes its decision from its own float64 values.  The GPU takes it
from float32 scores and a float64 history of float32 sums, so near a threshold
or a tie the two may legitimately differ.  A different GPU decision is accepted
only where the oracle's own margin lies inside the rounding bound stated here;
every other difference fails.  Pure numpy: usable on the CPU (see
tests/test_decisions.py, which plants wrong decisions and checks that each is
refused).
"""
from __future__ import annotations

import numpy as np

from oracle import plan

# Shares are ratios of float32 scores: the GPU's scores are the float32
# roundings (2^-24 relative) of float64 probabilities that agree with the
# oracle's to ~1e-15, so a share differs by at most ~(k + 1) 2^-24 relative.
SHARE_EPS = 1e-6
# Demand history: float64 sums of float32 scores against the oracle's float64
# sums of float64 scores -- within 1e-5 relative (the demand bar).
HIST_REL = 1e-5


def hist_close(a: float, b: float) -> bool:
    return abs(a - b) <= HIST_REL * max(abs(a), abs(b))


def check_hot_pick(got, te, ts, es, hist, n_arena, threshold=0.2):
    """got = (e_star, c) from the GPU (-1 = none).  Raises AssertionError unless
    it equals the oracle's decision or differs only inside the margins.
    Returns the oracle's decision (e_star, c) for reporting."""
    es = np.asarray(es)
    want = plan.hot_read(ts, te, es, hist, n_arena, threshold)
    w_e, w_c = (want[0], want[1]) if want is not None else (-1, None)
    arena = [e for e in range(es.shape[0]) if 0 <= es[e] < n_arena]
    if w_c is None:
        w_c = min(arena, key=lambda e: (hist[e], e)) if arena else -1
    g_e, g_c = int(got[0]), int(got[1])
    if (g_e, g_c) == (w_e, w_c):
        return w_e, w_c
    share = plan.pick_shares(ts)
    miss = np.asarray(es)[np.asarray(te)] < 0
    best = float(share[miss].max()) if miss.any() else -np.inf
    if g_e != w_e:
        if g_e < 0:
            # the GPU found no candidate: the oracle's best must sit at the threshold
            assert best < threshold + SHARE_EPS, ("GPU found no hot read", w_e, best)
        else:
            rows = (np.asarray(te) == g_e) & miss
            assert rows.any(), ("GPU's e* is not a miss of this batch", g_e)
            g_best = float(share[rows].max())
            assert g_best >= threshold - SHARE_EPS, ("GPU's e* below the threshold", g_e, g_best)
            assert g_best >= best - SHARE_EPS, ("GPU's e* is not (near) the heaviest miss",
                                                g_e, g_best, w_e, best)
    if g_c != w_c:
        assert g_c in arena, ("GPU's c is not an arena expert", g_c)
        # a zero history is exact on both sides: a tie at zero goes to the lower id
        assert hist[w_c] != 0 or hist[g_c] != 0, ("tie at zero broken differently", g_c, w_c)
        assert hist_close(hist[g_c], hist[w_c]), \
            ("GPU's c is not (near) the coldest", g_c, hist[g_c], w_c, hist[w_c])
    return w_e, w_c


def check_replan(got_ev, got_ld, got_table, hist, table, n_swap, k):
    """The GPU's re-plan (evicted list, loaded list, new table) against the
    oracle's on the oracle's float64 history.  Equal, or each list's sorted
    history values within HIST_REL of the oracle's, every constraint held, and
    the table the lists imply.  Returns the oracle's (evicted, loaded, table)."""
    hist = np.asarray(hist, dtype=np.float64)
    table = np.asarray(table)
    oev, old, onew = plan.replan(hist, table, n_swap, k)
    got_ev = [tuple(map(int, p)) for p in got_ev]
    got_ld = [tuple(map(int, p)) for p in got_ld]
    if got_ev == [tuple(p) for p in oev] and got_ld == [tuple(p) for p in old]:
        assert np.array_equal(got_table, onew), "same lists, different table"
        return oev, old, onew
    assert len(got_ev) == len(oev) and len(got_ld) == len(old), "swap counts differ"
    assert len(set(got_ev)) == len(got_ev) and len(set(got_ld)) == len(got_ld)
    for l, e in got_ev:
        assert table[l, e] >= 0, ("evicted a non-resident pair", l, e)
    for l, e in got_ld:
        assert table[l, e] < 0, ("loaded a resident pair", l, e)
    for gv, wv in zip(sorted(hist[l, e] for l, e in got_ev), sorted(hist[l, e] for l, e in oev)):
        assert hist_close(gv, wv), ("evictions differ beyond the margin", gv, wv)
    for gv, wv in zip(sorted(hist[l, e] for l, e in got_ld), sorted(hist[l, e] for l, e in old)):
        assert hist_close(gv, wv), ("loads differ beyond the margin", gv, wv)
    # a zero history is exact on both sides: pairs at zero follow the (l, e) order
    for got, want in ((got_ev, oev), (got_ld, old)):
        gz = [p for p in got if hist[p] == 0]
        wz = [tuple(p) for p in want if hist[tuple(p)] == 0]
        assert gz == wz, ("pairs with zero history chosen differently", gz[:5], wz[:5])
    # the table the GPU's lists imply, and the per-layer floor
    new = table.copy()
    for (le, ee), (ll, el) in zip(got_ev, got_ld):
        new[ll, el] = table[le, ee]
        new[le, ee] = -1
    assert np.array_equal(got_table, new), "table does not follow the swap lists"
    floor = np.minimum((table >= 0).sum(axis=1), k)
    assert ((new >= 0).sum(axis=1) >= floor).all(), "a layer fell below k routable experts"
    return oev, old, onew


def check_ring_plan(got, weight, table, ring, head, per_step, slot0):
    """The GPU's ring picks [(r, l, e)] against the oracle's ring_plan on the
    oracle's float64 step demand.  Equal, or the picked pairs' weights, in
    order, within HIST_REL of the oracle's (float32 per-call demand against
    float64 sums), every pick a valid candidate, entries in ring order.
    Returns the plan to continue the simulation with (the GPU's, once accepted)
    as (plan, table, ring, head) after applying it."""
    want = plan.ring_plan(weight, table, ring, head, per_step, slot0)
    got = [tuple(int(v) for v in p) for p in got]
    if got == [tuple(p) for p in want[0]]:
        return want
    w = np.asarray(weight, dtype=np.float64)
    tab = np.asarray(table)
    L, E = tab.shape
    assert len(got) == len(want[0]), ("ring pick counts differ", got, want[0])
    in_ring = {p for p in ring if p >= 0}
    R = len(ring)
    for i, (r, l, e) in enumerate(got):
        assert r == (head + i) % R, ("ring entries out of order", got)
        assert tab[l, e] < 0 and w[l, e] > 0 and l * E + e not in in_ring, ("not a miss", l, e)
    assert len({(l, e) for _, l, e in got}) == len(got)
    for (_, gl, ge), (_, wl, we) in zip(got, want[0]):
        assert hist_close(w[gl, ge], w[wl, we]), ("ring picks differ beyond the margin",
                                                  (gl, ge, w[gl, ge]), (wl, we, w[wl, we]))
    # apply the GPU's picks with the oracle's eviction rule
    tab = tab.copy()
    ring = list(ring)
    for r, l, e in got:
        old = ring[r]
        if old >= 0 and tab[old // E, old % E] == slot0 + r:
            tab[old // E, old % E] = -1
        ring[r] = l * E + e
    return got, tab, ring, (head + len(got)) % R
