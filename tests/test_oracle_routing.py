"""Pins for the oracle's routing steps O1-O8 (CPU only).

Checked against correctly rounded sums (math.fsum), brute-force sorting with
explicit key tuples, a literal implementation of "a missing pick is replaced by
the next-best resident one" (TideLM README, "How adaptive expert loading
works", item 2), the demand invariants of item 1, and the hand-worked example
in tests/golden/routing_worked.txt.
"""
import itertools
import math
import os

import numpy as np
import pytest

import fixtures
from oracle import moe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "routing_worked.txt")


def _small(T=5, H=64, E=9, seed=3, bias=0.3):
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=3, I=32, n_routable=E, seed=seed, bias_scale=bias)
    return lay


# --- O1 ---------------------------------------------------------------------
def check_logits_fsum():
    for seed in range(4):
        lay = _small(seed=seed)
        z = moe.router_logits(lay.x_bits, lay.w_router, lay.bias)
        x = fixtures.bf16_bits_to_f32(lay.x_bits).astype(np.float64)
        w = lay.w_router.astype(np.float64)
        for t in range(x.shape[0]):
            for e in range(w.shape[0]):
                terms = [float(a) * float(b) for a, b in zip(x[t], w[e])] + [float(lay.bias[e])]
                exact = math.fsum(terms)
                assert abs(z[t, e] - exact) <= math.ulp(exact) * 4 + 1e-300, (t, e, z[t, e], exact)


def test_logits_match_correctly_rounded_sum():
    check_logits_fsum()


# --- O2 / O7 -----------------------------------------------------------------
def check_softmax_and_renorm():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((20, 12)) * 3
    p = moe.softmax(z)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-15, rtol=0)
    for t in range(20):
        ref = [math.exp(v) for v in z[t]]
        s = math.fsum(ref)
        assert np.allclose(p[t], np.array(ref) / s, rtol=1e-13, atol=0)
    es = np.arange(12, dtype=np.int32)
    es[[1, 4, 7]] = -1
    picks = moe.masked_topk(z, es, 4)
    w = moe.renormalise(p, picks)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15, rtol=0)
    for t in range(20):
        ez = [math.exp(z[t, e]) for e in picks[t]]
        assert np.allclose(w[t], np.array(ez) / math.fsum(ez), rtol=1e-13, atol=0)
    w1 = moe.renormalise(p, moe.masked_topk(z, es, 1))
    assert (w1[:, 0] == 1.0).all()


def test_softmax_and_renormalisation():
    check_softmax_and_renorm()


# --- O3 / O6 -----------------------------------------------------------------
def brute_topk(zrow, allowed, k):
    cand = [e for e in range(len(zrow)) if allowed[e]]
    cand.sort(key=lambda e: (-zrow[e], e))
    got = sorted(cand[:k])
    return got + [-1] * (k - len(got))


def check_topk_bruteforce():
    rng = np.random.default_rng(5)
    for trial in range(200):
        E = int(rng.integers(2, 12))
        k = int(rng.integers(1, E + 1))
        z = rng.integers(-3, 4, size=(4, E)).astype(np.float64) * 0.5   # many ties
        allowed = rng.random(E) < 0.6
        es = np.where(allowed, np.arange(E), -1)
        u = moe.topk(z, k)
        m = moe.masked_topk(z, es, k)
        for t in range(4):
            assert list(u[t]) == brute_topk(z[t], np.ones(E, bool), k)
            assert list(m[t]) == brute_topk(z[t], allowed, k)


def test_topk_bruteforce_with_ties():
    check_topk_bruteforce()


def test_all_equal_logits_pick_lowest_ids():
    z = np.zeros((3, 10))
    assert (moe.topk(z, 4) == np.arange(4)).all()


def test_all_resident_mask_equals_plain_topk():
    lay = _small(T=16, E=16, seed=9)
    r_all = moe.route(lay.x_bits, lay.w_router, lay.bias, np.arange(16, dtype=np.int32), 4)
    assert np.array_equal(r_all["sel_expert"], r_all["topk_expert"])
    p_u = moe.gather(r_all["p"], r_all["topk_expert"])
    assert np.allclose(r_all["sel_weight"], p_u / p_u.sum(axis=1, keepdims=True), rtol=1e-15)


def literal_replacement(zrow, allowed, k):
    """Item 2 read literally: take the wanted top-k; each miss, best first, is
    replaced by the best resident expert not already picked."""
    order = sorted(range(len(zrow)), key=lambda e: (-zrow[e], e))
    wanted = order[:k]
    picked = [e for e in wanted if allowed[e]]
    for miss in [e for e in wanted if not allowed[e]]:
        for e in order:
            if allowed[e] and e not in picked:
                picked.append(e)
                break
    got = sorted(picked)
    return got + [-1] * (k - len(got))


def check_replacement_equivalence():
    rng = np.random.default_rng(1)
    for E in (4, 6, 8):
        for k in range(1, E + 1, 2):
            z = rng.integers(-2, 3, size=(6, E)).astype(np.float64)
            for mask in itertools.product([False, True], repeat=E):
                allowed = np.array(mask)
                es = np.where(allowed, np.arange(E), -1)
                m = moe.masked_topk(z, es, k)
                for t in range(z.shape[0]):
                    assert list(m[t]) == literal_replacement(z[t], allowed, k), (E, k, mask, t)


def test_masked_topk_equals_literal_miss_replacement():
    check_replacement_equivalence()


# --- O4 ----------------------------------------------------------------------
def check_demand():
    lay = _small(T=40, E=12, seed=4)
    z = moe.router_logits(lay.x_bits, lay.w_router, lay.bias)
    p = moe.softmax(z)
    te = moe.topk(z, 3)
    ts = moe.gather(p, te)
    d = moe.demand(te, ts, 12)
    d2 = moe.demand_fast(te, ts, 12)
    assert np.array_equal(d, d2)
    total = math.fsum(float(p[t, e]) for t in range(40) for e in te[t])
    assert abs(d.sum() - total) <= 1e-13 * total
    for e in range(12):
        want = math.fsum(float(p[t, e]) for t in range(40) if e in te[t])
        assert abs(d[e] - want) <= 1e-14 * max(want, 1e-300)
    # k = E and no bias: every token contributes its whole distribution
    dk = moe.demand(moe.topk(z, 12), moe.gather(p, moe.topk(z, 12)), 12)
    assert abs(dk.sum() - 40) < 1e-12


def test_demand_invariants():
    check_demand()


def test_demand_independent_of_mask():
    lay = _small(T=30, E=10, seed=8)
    deltas = []
    for mask_seed in range(5):
        es = np.where(np.random.default_rng(mask_seed).random(10) < 0.5, np.arange(10), -1)
        es[0] = 0
        r = moe.route(lay.x_bits, lay.w_router, lay.bias, es.astype(np.int32), 3)
        deltas.append(moe.demand(r["topk_expert"], r["topk_score"], 10))
    for d in deltas[1:]:
        assert np.array_equal(d, deltas[0])


# --- O8 ----------------------------------------------------------------------
def brute_bucket(sel_slot, S):
    flat = list(np.asarray(sel_slot).reshape(-1))
    perm, counts = [], []
    for s in range(S):
        mine = [a for a, v in enumerate(flat) if v == s]
        counts.append(len(mine))
        perm += mine
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    return counts, offsets, perm + [-1] * (len(flat) - len(perm))


def check_bucket():
    rng = np.random.default_rng(2)
    for trial in range(50):
        T, k, S = int(rng.integers(1, 30)), int(rng.integers(1, 6)), int(rng.integers(1, 12))
        ss = rng.integers(-1, S, size=(T, k))
        c, o, p = moe.bucket(ss, S)
        bc, bo, bp = brute_bucket(ss, S)
        assert list(c) == bc and list(o) == bo and list(p) == bp
        valid = p[p >= 0]
        assert sorted(valid) == sorted(np.flatnonzero(ss.reshape(-1) >= 0))


def test_bucket_bruteforce():
    check_bucket()


# --- worked example ----------------------------------------------------------
def _golden():
    d = {}
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            key, val = [s.strip() for s in line.split("|")]
            rows = [[float(v) if "." in v else int(v) for v in r.split(",")] for r in val.split(";")]
            d[key] = rows
    return d


def test_worked_example():
    g = _golden()
    E, H, k = 6, 32, 3
    w = np.zeros((E, H), dtype=np.float32)
    w[:, 0] = g["W0"][0]
    w[:, 1] = g["W1"][0]
    x = np.zeros((2, H), dtype=np.float32)
    x[0, 0] = 1.0
    x[1, 1] = 1.0
    es = np.array(g["expert_slot"][0], dtype=np.int32)
    r = moe.route(fixtures.f32_to_bf16_bits(x), w, None, es, k)
    assert r["topk_expert"].tolist() == g["topk_expert"]
    assert r["sel_expert"].tolist() == g["sel_expert"]
    assert r["sel_slot"].tolist() == g["sel_slot"]
    c, o, p = moe.bucket(r["sel_slot"], 4)
    assert o.tolist() == g["offsets"][0]
    assert p.tolist() == g["perm"][0]
    e1, e2, e15 = math.exp(1), math.exp(2), math.exp(1.5)
    s0 = e1 + e2 + e15
    assert np.allclose(r["sel_weight"][0], [e1 / s0, e2 / s0, e15 / s0], rtol=1e-15)
    s1 = math.exp(3) + 1 + math.exp(1)
    assert np.allclose(r["sel_weight"][1], [math.exp(3) / s1, 1 / s1, math.exp(1) / s1], rtol=1e-15)
    z0 = [0.5, 2.0, 1.0, 2.0, -1.0, 1.5]
    z1 = [3.0, 0.0, 0.0, 1.0, 2.5, -2.0]
    p0 = [math.exp(v) / math.fsum(math.exp(u) for u in z0) for v in z0]
    p1 = [math.exp(v) / math.fsum(math.exp(u) for u in z1) for v in z1]
    d = moe.demand(r["topk_expert"], r["topk_score"], E)
    want = [p1[0], p0[1], 0.0, p0[3] + p1[3], p1[4], p0[5]]
    assert np.allclose(d, want, rtol=1e-14, atol=0)
