"""Host decisions around the layer: hot read and arena re-plan -- oracle side.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

hot_read follows the TideLM README's "How adaptive expert loading works",
item 3, GLM-5.3 bullet: a layer's heaviest miss carrying at least 0.2 of a
token's routing weight is read before that layer's experts run and is kept in
place of the coldest expert.  replan follows item 1: one arena is shared by
all layers, re-planned from the demand history, so a busy layer takes slots
from a quiet one.
"""
from __future__ import annotations

import numpy as np


def pick_shares(topk_score: np.ndarray) -> np.ndarray:
    """share[t,j] = score[t,j] / sum over the token's unrestricted picks.

    The scores are the recorded float32 routing scores; the arithmetic is
    float64 with the sum taken in ascending pick order, so that the >= 0.2
    decision is taken in one stated precision on every implementation.
    """
    v = np.asarray(topk_score, dtype=np.float32).astype(np.float64)
    s = np.zeros(v.shape[0], dtype=np.float64)
    for j in range(v.shape[1]):
        s = s + v[:, j]
    return v / s[:, None]


def hot_read(topk_score, topk_expert, expert_slot, hist_after, n_arena, threshold=0.2):
    """O12.  Returns (e_star, c, new_expert_slot) or None when no miss qualifies.

    e_star: the non-routable expert with the largest share >= threshold over
    all tokens (ties: lower expert id, then lower token).  c: the arena-resident
    expert (slot < n_arena; hot-ring slots excluded) with the smallest demand
    history, ties to the lower id.  e_star takes c's slot; c becomes
    non-routable.
    """
    es = np.asarray(expert_slot)
    share = pick_shares(topk_score)
    best = None  # (share, -e, -t) maximised
    T, k = topk_expert.shape
    for t in range(T):
        for j in range(k):
            e = int(topk_expert[t, j])
            if es[e] >= 0 or share[t, j] < threshold:
                continue
            key = (share[t, j], -e, -t)
            if best is None or key > best:
                best = key
    if best is None:
        return None
    e_star = -best[1]
    arena = [e for e in range(es.shape[0]) if 0 <= es[e] < n_arena]
    c = min(arena, key=lambda e: (hist_after[e], e))
    new = es.copy()
    new[e_star] = es[c]
    new[c] = -1
    return e_star, c, new


def replan(hist: np.ndarray, expert_slot: np.ndarray, n_swap: int, k: int):
    """O13 over a [L,E] demand history and [L,E] slot table.

    Evict the n_swap resident (l,e) with the smallest history (ties: lower
    (l,e)), skipping any eviction that would leave a layer with fewer than k
    routable experts; load the n_swap non-resident (l,e) with the largest
    history (ties: lower (l,e)).  The i-th evicted slot receives the i-th
    loaded pair.  Returns (evicted list, loaded list, new slot table).
    """
    hist = np.asarray(hist, dtype=np.float64)
    es = np.asarray(expert_slot)
    L, E = es.shape
    res = [(hist[l, e], l, e) for l in range(L) for e in range(E) if es[l, e] >= 0]
    non = [(-hist[l, e], l, e) for l in range(L) for e in range(E) if es[l, e] < 0]
    res.sort()
    non.sort()
    count = (es >= 0).sum(axis=1)
    evicted = []
    for _, l, e in res:
        if len(evicted) == n_swap:
            break
        if count[l] - 1 < k:
            continue
        count[l] -= 1
        evicted.append((l, e))
    loaded = [(l, e) for _, l, e in non[:len(evicted)]]
    new = es.copy()
    for (le, ee), (ll, el) in zip(evicted, loaded):
        new[ll, el] = es[le, ee]
        new[le, ee] = -1
    return evicted, loaded, new


# ----------------------------------------------------------------------------
# Hot ring (TideLM README, "How adaptive expert loading works", item 3,
# DeepSeek bullet, and "Settings worth knowing": the ring's slots sit on top
# of the arena budget).  After each step the heaviest misses of that step --
# every lane's tokens feed one plan -- are read into ring slots of their own
# while the next step runs, and are routable from the step after it until the
# ring wraps round onto them.
#
# State: ring[r] = the pair id l*E + e held (or being filled) by ring entry r,
# -1 if empty; head = the entry the next pick overwrites.  Ring entry r is
# global slot slot0 + r.
# ----------------------------------------------------------------------------
def ring_plan(miss_weight, table, ring, head, per_step, slot0):
    """One step's ring plan.

    miss_weight [L][E]: the step's demand of every (layer, expert) -- the sum
    of the routing scores of the picks the router wanted (item 1's record for
    this step).  Candidates: pairs that are not routable (table < 0), are not
    already in the ring, and have weight > 0.  The first min(per_step, R) of
    them by (larger weight, then lower pair id) take ring entries head, head+1,
    ... (mod R) in that order.  The pair an entry held before is evicted: if
    the table routes it to that entry's slot it becomes non-routable at once
    (the copy will overwrite the slot), otherwise the table is left alone.
    The new pairs stay non-routable until ring_install.

    Returns (plan [(r, l, e)], new table, new ring, new head).
    """
    w = np.asarray(miss_weight, dtype=np.float64)
    tab = np.asarray(table).copy()
    L, E = tab.shape
    ring = list(int(v) for v in ring)
    R = len(ring)
    in_ring = {p for p in ring if p >= 0}
    cands = [(-w[l, e], l * E + e) for l in range(L) for e in range(E)
             if tab[l, e] < 0 and w[l, e] > 0 and l * E + e not in in_ring]
    cands.sort()
    plan = []
    for i, (_, p) in enumerate(cands[:min(per_step, R)]):
        r = (head + i) % R
        old = ring[r]
        if old >= 0 and tab[old // E, old % E] == slot0 + r:
            tab[old // E, old % E] = -1
        ring[r] = p
        plan.append((r, p // E, p % E))
    return plan, tab, ring, (head + len(plan)) % R if R else 0


def ring_install(plan, table, ring, slot0):
    """Make a plan's pairs routable once their bytes are in place: each
    (r, l, e) whose ring entry still holds (l, e) gets table[l, e] = slot0 + r
    (an entry taken over by a later plan meanwhile is skipped)."""
    tab = np.asarray(table).copy()
    L, E = tab.shape
    for r, l, e in plan:
        if ring[r] == l * E + e:
            tab[l, e] = slot0 + r
    return tab
