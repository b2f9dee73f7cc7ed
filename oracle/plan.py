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


# ----------------------------------------------------------------------------
# Demand-history planner (TideLM README, "How adaptive expert loading works",
# item 1: the history persists across restarts, the arena is filled from it at
# boot and re-planned after each prompt's prefill, every few hundred generated
# tokens and between requests; "Settings worth knowing": a sensitivity setting
# sets how fast the resident set follows new traffic, and GLM_ADAPT_EVERY=200
# the re-plan period in generated tokens).
# ----------------------------------------------------------------------------
def boot_fill(hist, n_slots, k):
    """Resident set and slot table filled from a history at boot.

    Every layer first keeps its min(k, E) hottest experts (so routing always
    finds k picks); the remaining slots go to the hottest remaining pairs.  A
    pair's place is (larger history, then its rank inside its layer, then
    lower layer), so equal histories -- a fresh, all-zero history above all --
    are shared round-robin between layers instead of filling layer 0 first.
    Within a layer, rank = position by (larger history, lower expert id).
    Slots 0, 1, ... go to the chosen pairs in ascending (layer, expert).
    Returns the [L][E] table (-1 = not resident)."""
    h = np.asarray(hist, dtype=np.float64)
    L, E = h.shape
    floor = min(k, E)
    if n_slots < L * floor:
        raise ValueError("fewer slots than the per-layer floor needs")
    n_slots = min(n_slots, L * E)
    rank = np.zeros((L, E), dtype=np.int64)
    for l in range(L):
        order = sorted(range(E), key=lambda e: (-h[l, e], e))
        for r, e in enumerate(order):
            rank[l, e] = r
    chosen = {(l, e) for l in range(L) for e in range(E) if rank[l, e] < floor}
    rest = sorted(((-h[l, e], rank[l, e], l, e) for l in range(L) for e in range(E)
                   if (l, e) not in chosen))
    for _, _, l, e in rest[:n_slots - len(chosen)]:
        chosen.add((l, e))
    table = np.full((L, E), -1, dtype=np.int64)
    for s, (l, e) in enumerate(sorted(chosen)):
        table[l, e] = s
    return table


SENSITIVITY_DECAY = {"low": 1.0, "medium": 0.9, "high": 0.75}


def decay(hist, factor):
    """History after forgetting: every entry times `factor` (applied before
    each re-plan, so older traffic weighs less; factor 1 keeps everything)."""
    return np.asarray(hist, dtype=np.float64) * float(factor)


def gainful_swaps(hist, evicted, loaded):
    """How many leading swaps of a re-plan gain demand: the i-th swap is kept
    while the pair it loads has a larger history than the pair it evicts (the
    lists run coldest-evicted and hottest-loaded first, so the gains only
    shrink along them)."""
    h = np.asarray(hist, dtype=np.float64)
    n = 0
    for ev, ld in zip(evicted, loaded):
        if not h[tuple(ld)] > h[tuple(ev)]:
            break
        n += 1
    return n


def replan_points(events, every):
    """Where the cadence re-plans, for a stream of serving events.

    events: ("prefill", request), ("token", request) per generated token, and
    ("end", request).  A re-plan follows each prefill; during decoding, every
    `every` generated tokens since the last re-plan; and at the end of a
    request when tokens were generated since the last one (between requests).
    Returns the indices of the events after which a re-plan runs."""
    out, since = [], 0
    for i, (kind, _) in enumerate(events):
        if kind == "prefill":
            out.append(i)
            since = 0
        elif kind == "token":
            since += 1
            if since >= every:
                out.append(i)
                since = 0
        elif kind == "end":
            if since > 0:
                out.append(i)
            since = 0
        else:
            raise ValueError(kind)
    return out
