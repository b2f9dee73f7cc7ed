"""Pins for the host decisions: hot read (O12) and arena re-plan (O13). CPU only.

Constructed cases with known answers and brute force over small tables.
"""
import numpy as np

from oracle import plan


def scores(p, te):
    return np.take_along_axis(p, te, axis=1).astype(np.float32)


def test_pick_shares_sum_in_order():
    ts = np.array([[0.25, 0.5, 0.25], [1.0, 0.0, 0.0]], dtype=np.float32)
    s = plan.pick_shares(ts)
    assert np.array_equal(s, [[0.25, 0.5, 0.25], [1.0, 0.0, 0.0]])


def test_hot_read_planted_miss():
    E, k = 8, 2
    p = np.full((3, E), 0.01)
    p[1, 5] = 0.5     # token 1 wants expert 5 (not resident) with share > 0.2
    p[1, 0] = 0.4
    p[0, 2] = 0.3
    p[0, 3] = 0.3
    p[2, 6] = 0.9
    p[2, 7] = 0.05
    p /= p.sum(axis=1, keepdims=True)
    te = np.array([[2, 3], [0, 5], [6, 7]])
    es = np.array([0, 1, 2, 3, -1, -1, 4, -1])
    hist = np.array([5.0, 0.5, 0.5, 2.0, 0, 0, 1.0, 0])
    r = plan.hot_read(scores(p, te), te, es, hist, n_arena=5)
    assert r is not None
    e_star, c, new = r
    # expert 7 is a miss too but its share (0.05/0.95) is below 0.2
    assert e_star == 5
    assert c == 1                      # ties at 0.5 between experts 1 and 2 -> lower id
    assert new[5] == 1 and new[1] == -1 and (new[[0, 2, 3, 6]] == es[[0, 2, 3, 6]]).all()


def test_hot_read_none_below_threshold():
    p = np.array([[0.4, 0.35, 0.25]])
    te = np.array([[0, 1]])
    es = np.array([0, -1, 1])
    # share of expert 1 = 0.35/0.75 = 0.467 > 0.2 -> one candidate
    assert plan.hot_read(scores(p, te), te, es, np.zeros(3), 2)[0] == 1
    p = np.array([[0.9, 0.1, 0.0]])
    te = np.array([[0, 1]])
    es = np.array([0, -1, -1])
    p2 = np.array([[0.95, 0.05, 0.0]])
    assert plan.hot_read(scores(p2, te), te, es, np.zeros(3), 1) is None   # share 0.05 < 0.2
    assert plan.hot_read(scores(p, te), te, es, np.zeros(3), 1) is None    # share 0.1


def test_hot_read_share_tie_breaks():
    # two misses with the same share: lower expert id wins; same expert: lower token
    te = np.array([[0, 3], [0, 2], [1, 3]])
    ts = np.array([[0.5, 0.5], [0.5, 0.5], [0.5, 0.5]], dtype=np.float32)
    es = np.array([0, 1, -1, -1])
    e_star, c, _ = plan.hot_read(ts, te, es, np.array([1.0, 0.5, 0, 0]), n_arena=2)
    assert e_star == 2 and c == 1


def test_hot_read_ring_slots_never_evicted():
    p = np.array([[0.5, 0.5, 0.0, 0.0]])
    te = np.array([[0, 1]])
    es = np.array([-1, 2, 0, 1])         # slot 2 is a ring slot (n_arena = 2)
    hist = np.array([0.0, 0.0, 3.0, 4.0])  # expert 1 is coldest but lives in the ring
    e_star, c, new = plan.hot_read(scores(p, te), te, es, hist, n_arena=2)
    assert e_star == 0 and c == 2


def brute_replan(hist, es, n, k):
    L, E = es.shape
    res = sorted(((hist[l, e], l, e) for l in range(L) for e in range(E) if es[l, e] >= 0))
    out = []
    cnt = {l: int((es[l] >= 0).sum()) for l in range(L)}
    for h, l, e in res:
        if len(out) < n and cnt[l] > k:
            out.append((l, e))
            cnt[l] -= 1
    non = sorted(((-hist[l, e], l, e) for l in range(L) for e in range(E) if es[l, e] < 0))
    return out, [(l, e) for _, l, e in non[:len(out)]]


def test_replan_bruteforce_and_floor():
    rng = np.random.default_rng(3)
    for trial in range(40):
        L, E, k = 3, 6, 2
        es = np.full((L, E), -1)
        slots = iter(range(100))
        for l in range(L):
            for e in rng.choice(E, size=int(rng.integers(2, 6)), replace=False):
                es[l, e] = next(slots)
        hist = rng.integers(0, 4, size=(L, E)).astype(float)   # many ties
        n = int(rng.integers(1, 5))
        ev, ld, new = plan.replan(hist, es, n, k)
        bev, bld = brute_replan(hist, es, n, k)
        assert ev == bev and ld == bld
        assert ((new >= 0).sum(axis=1) >= np.minimum((es >= 0).sum(axis=1), k)).all()
        assert sorted(new[new >= 0]) == sorted(es[es >= 0])   # slots are conserved
        for (le, ee), (ll, el) in zip(ev, ld):
            assert new[ll, el] == es[le, ee]


def test_replan_hand_worked():
    """Two layers of four experts, worked by hand.

    Resident: layer 0 experts 0, 1, 2 (slots 0, 1, 2); layer 1 experts 0, 1
    (slots 3, 4).  Histories: layer 0 [5, 1, 0.5, 8], layer 1 [0.25, 3, 6, 8].
    Residents by ascending history: (1,0) 0.25, (0,2) 0.5, (0,1) 1, (1,1) 3,
    (0,0) 5.  Non-residents by descending history: (0,3) 8, (1,3) 8 (tie: lower
    layer first), (1,2) 6.
    """
    table = np.array([[0, 1, 2, -1], [3, 4, -1, -1]])
    hist = np.array([[5.0, 1.0, 0.5, 8.0], [0.25, 3.0, 6.0, 8.0]])
    # k = 2: (1,0) would leave layer 1 with one expert -> skipped; (0,2) is
    # taken; then layer 0 is at two and layer 1 at two: nothing else can go.
    ev, ld, new = plan.replan(hist, table, 2, 2)
    assert ev == [(0, 2)] and ld == [(0, 3)]
    assert new.tolist() == [[0, 1, -1, 2], [3, 4, -1, -1]]
    # k = 1: (1,0) then (0,2) are evicted; (0,3) takes slot 3 (layer 1's, a
    # slot moving between layers) and (1,3) takes slot 2 (layer 0's).
    ev, ld, new = plan.replan(hist, table, 2, 1)
    assert ev == [(1, 0), (0, 2)] and ld == [(0, 3), (1, 3)]
    assert new.tolist() == [[0, 1, -1, 3], [-1, 4, -1, 2]]
    # asking for more swaps than the floor allows stops at what can move
    ev, ld, new = plan.replan(hist, table, 5, 1)
    assert ev == [(1, 0), (0, 2), (0, 1)] and ld == [(0, 3), (1, 3), (1, 2)]
    assert new.tolist() == [[0, -1, -1, 3], [-1, 4, 1, 2]]


# ---------------------------------------------------------------------------
# hot ring
# ---------------------------------------------------------------------------
def test_ring_hand_worked():
    """Two layers of four experts, a ring of 3 entries (global slots 10-12),
    two picks a step; worked by hand."""
    table = np.array([[0, -1, 1, -1], [2, -1, -1, -1]])
    w = np.array([[0.5, 0.3, 0.9, 0.0], [0.2, 0.3, 0.7, 0.1]])
    # misses: (0,1) 0.3, (1,1) 0.3, (1,2) 0.7, (1,3) 0.1; (0,3) has no weight.
    # heaviest first, the 0.3 tie to the lower pair id (0,1) = 1 before (1,1) = 5
    plan_a, t1, ring, head = plan.ring_plan(w, table, [-1, -1, -1], 0, 2, 10)
    assert plan_a == [(0, 1, 2), (1, 0, 1)] and ring == [6, 1, -1] and head == 2
    assert np.array_equal(t1, table)              # nothing routable before the install
    t2 = plan.ring_install(plan_a, t1, ring, 10)
    assert t2.tolist() == [[0, 11, 1, -1], [2, -1, 10, -1]]
    # next step: (1,1) takes the empty entry 2, (1,3) wraps onto entry 0 and
    # evicts (1,2), which stops being routable at once
    plan_b, t3, ring, head = plan.ring_plan(w, t2, ring, head, 2, 10)
    assert plan_b == [(2, 1, 1), (0, 1, 3)] and ring == [7, 1, 5] and head == 1
    assert t3.tolist() == [[0, 11, 1, -1], [2, -1, -1, -1]]
    t4 = plan.ring_install(plan_b, t3, ring, 10)
    assert t4.tolist() == [[0, 11, 1, -1], [2, 12, -1, 10]]


def test_ring_pending_pairs_not_planned_twice_and_stale_install_skipped():
    table = np.array([[-1, -1, 0]])
    w = np.array([[0.4, 0.6, 0.9]])
    p1, t1, ring, head = plan.ring_plan(w, table, [-1], 0, 1, 5)
    assert p1 == [(0, 0, 1)] and ring == [1]
    # planned again before the install: expert 1 is in flight, so expert 0 is
    # next, and it takes the only entry over
    p2, t2, ring, head = plan.ring_plan(w, t1, ring, head, 1, 5)
    assert p2 == [(0, 0, 0)] and ring == [0]
    t3 = plan.ring_install(p1, t2, ring, 5)       # entry 0 no longer holds expert 1
    assert t3.tolist() == [[-1, -1, 0]]
    t4 = plan.ring_install(p2, t3, ring, 5)
    assert t4.tolist() == [[5, -1, 0]]


def brute_ring_picks(w, table, ring, per_step):
    """Literal "take the heaviest remaining miss" rounds (no sort)."""
    L, E = table.shape
    taken = set(p for p in ring if p >= 0)
    out = []
    for _ in range(min(per_step, len(ring))):
        best = None
        for l in range(L):
            for e in range(E):
                p = l * E + e
                if table[l, e] >= 0 or w[l, e] <= 0 or p in taken:
                    continue
                if best is None or w[l, e] > w[best // E, best % E]:
                    best = p       # strict: an equal weight later in the scan loses
        if best is None:
            break
        taken.add(best)
        out.append(best)
    return out


def test_ring_bruteforce_and_invariants():
    rng = np.random.default_rng(8)
    for trial in range(60):
        L, E, R = int(rng.integers(1, 4)), int(rng.integers(2, 9)), int(rng.integers(1, 6))
        slot0 = 100
        table = np.where(rng.random((L, E)) < 0.4, 0, -1)
        table[table >= 0] = np.arange(int((table >= 0).sum()))
        ring, head = [-1] * R, 0
        pending = []
        for step in range(6):
            w = rng.integers(0, 4, size=(L, E)) / 4.0        # ties and zeros
            per = int(rng.integers(1, R + 1))
            want = brute_ring_picks(w, table, ring, per)
            p, t2, ring2, head2 = plan.ring_plan(w, table, ring, head, per, slot0)
            assert [l * E + e for _, l, e in p] == want
            assert [r for r, _, _ in p] == [(head + i) % R for i in range(len(p))]
            assert head2 == (head + len(p)) % R
            live = [q for q in ring2 if q >= 0]
            assert len(live) == len(set(live))             # a pair is in the ring once
            for r, q in enumerate(ring2):                   # routable ring pairs use their slot
                if q >= 0 and t2[q // E, q % E] >= slot0:
                    assert t2[q // E, q % E] == slot0 + r
            for r, q in enumerate(ring):                    # evicted pairs are not routable
                if q >= 0 and q not in live:
                    assert t2[q // E, q % E] != slot0 + r
            table, ring, head = t2, ring2, head2
            pending.append(p)
            if len(pending) == 2:                           # installed one step later
                table = plan.ring_install(pending.pop(0), table, ring, slot0)
