"""The margin rules of tests/decisions.py refuse wrong decisions and accept
only differences inside the stated rounding bounds (CPU)."""
import numpy as np
import pytest

from decisions import HIST_REL, check_hot_pick, check_replan
from oracle import plan


def _hot_case():
    # 3 tokens, k = 2, 6 experts; experts 4 and 5 are not routable
    te = np.array([[0, 4], [1, 5], [2, 3]])
    ts = np.array([[0.5, 0.5], [0.7, 0.3], [0.6, 0.4]])
    es = np.array([0, 1, 2, 3, -1, -1])
    hist = np.array([3.0, 1.0, 2.0, 5.0, 0.0, 0.0])
    return te, ts, es, hist


def test_hot_pick_equal_accepted():
    te, ts, es, hist = _hot_case()
    assert check_hot_pick((4, 1), te, ts, es, hist, n_arena=4) == (4, 1)


@pytest.mark.parametrize("got", [(5, 1), (4, 0), (4, 3), (-1, 1), (0, 1), (4, 4)])
def test_hot_pick_wrong_refused(got):
    te, ts, es, hist = _hot_case()
    with pytest.raises(AssertionError):
        check_hot_pick(got, te, ts, es, hist, n_arena=4)


def test_hot_pick_near_tie_accepted():
    te, ts, es, hist = _hot_case()
    # expert 5's share a hair under expert 4's: either answer is within rounding
    ts = ts.copy()
    ts[1] = [0.5 + 2e-7, 0.5 - 2e-7]
    ts[0] = [0.5, 0.5]
    want = plan.hot_read(ts, te, es, hist, 4)
    assert want[0] == 4
    check_hot_pick((5, 1), te, ts, es, hist, n_arena=4)
    # the coldest arena expert within the history bound
    h2 = hist.copy()
    h2[0] = h2[1] * (1 + 0.5 * HIST_REL)
    check_hot_pick((4, 0), te, ts, es, h2, n_arena=4)


def test_hot_pick_threshold_margin():
    te, ts, es, hist = _hot_case()
    # the best miss sits at the threshold: "none" is within rounding
    thr = float(plan.pick_shares(ts)[0, 1])
    check_hot_pick((-1, 1), te, ts, es, hist, n_arena=4, threshold=thr)
    with pytest.raises(AssertionError):
        check_hot_pick((-1, 1), te, ts, es, hist, n_arena=4, threshold=thr - 1e-3)


def test_hot_pick_zero_tie_must_match():
    te, ts, es, hist = _hot_case()
    hist = np.array([0.0, 0.0, 2.0, 5.0, 0.0, 0.0])
    check_hot_pick((4, 0), te, ts, es, hist, n_arena=4)
    with pytest.raises(AssertionError):
        check_hot_pick((4, 1), te, ts, es, hist, n_arena=4)


def _replan_case():
    table = np.array([[0, 1, 2, -1, -1], [3, 4, -1, -1, 5]])
    hist = np.array([[4.0, 0.5, 2.0, 9.0, 0.0], [1.0, 3.0, 7.0, 0.0, 6.0]])
    return table, hist


def test_replan_equal_and_wrong():
    table, hist = _replan_case()
    ev, ld, new = plan.replan(hist, table, 2, 1)
    check_replan(ev, ld, new, hist, table, 2, 1)
    with pytest.raises(AssertionError):   # evicts a warmer pair
        bad = [ev[0], (1, 4)]
        t = table.copy()
        for (le, ee), (ll, el) in zip(bad, ld):
            t[ll, el] = table[le, ee]
            t[le, ee] = -1
        check_replan(bad, ld, t, hist, table, 2, 1)
    with pytest.raises(AssertionError):   # table does not follow the lists
        check_replan(ev, ld, table, hist, table, 2, 1)


def test_replan_near_tie_accepted():
    table, hist = _replan_case()
    hist = hist.copy()
    hist[1, 0] = hist[0, 1] * (1 + 0.5 * HIST_REL)   # two nearly equal coldest pairs
    ev, ld, new = plan.replan(hist, table, 1, 1)
    alt = [(1, 0)] if ev[0] == (0, 1) else [(0, 1)]
    t = table.copy()
    t[ld[0]] = table[alt[0]]
    t[alt[0]] = -1
    check_replan(alt, ld, t, hist, table, 1, 1)
