"""GPU parity of the hot read: moe_hot_pick against the oracle's decision, and
the whole hot-read layer call (route with demand, pick, copy into the coldest
expert's slot, re-route, experts) against the oracle run with the new table.

Bars: the decision (e*, c) and every routing output bit-exact; the slot's bytes
equal the loaded expert's packed bytes; output relative L2 within 5e-3.
"""
import numpy as np
import pytest

import fixtures
from oracle import moe, plan
from decisions import check_hot_pick
from gpu_helpers import GpuLayer, say, to_dev

pytestmark = pytest.mark.gpu

OUT_REL_L2 = 5e-3


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import resident_expert_routing_amd  # noqa: F401
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def gpu_pick(te, ts, es, hist, n_arena, threshold=0.2):
    import torch
    import resident_expert_routing_amd as m
    T, k = te.shape
    E = es.shape[0]
    S = int(es.max()) + 1 if (es >= 0).any() else 0
    out = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    need = m.moe_workspace_bytes(m.MOE_OP_HOT_PICK, T, 0, 0, 0, 0, 0)
    # stale partials from an earlier call must not leak into this one
    ws = torch.full((need + 256,), 0x7F, dtype=torch.uint8, device="cuda")
    m.check(m.moe_hot_pick(to_dev(te.astype(np.int32)) if T else None,
                           to_dev(ts.astype(np.float32)) if T else None, T, k, E,
                           to_dev(es.astype(np.int32)), S, n_arena, to_dev(hist.astype(np.float64)),
                           threshold, out, ws, need), "moe_hot_pick")
    torch.cuda.synchronize()
    return [int(v) for v in out.cpu()]


def oracle_pick(te, ts, es, hist, n_arena, threshold=0.2):
    r = plan.hot_read(ts, te, es, hist, n_arena, threshold)
    if r is None:
        return None
    return [r[0], r[1]]


def test_hot_pick_random_tables_with_ties():
    rng = np.random.default_rng(11)
    cases = 0
    for trial in range(60):
        T = int(rng.integers(1, 3000))
        E = int(rng.integers(4, 300))
        k = int(rng.integers(1, min(E, 32) + 1))
        te = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        te.sort(axis=1)
        # quantised scores give many equal shares
        ts = (rng.integers(1, 9, size=(T, k)) / 16.0).astype(np.float32)
        nres = int(rng.integers(1, E + 1))
        es = np.full(E, -1, dtype=np.int32)
        es[rng.choice(E, nres, replace=False)] = rng.permutation(nres)
        n_arena = int(rng.integers(1, nres + 1))    # slot 0 is always an arena slot
        hist = rng.integers(0, 4, size=E).astype(np.float64)
        thr = float(rng.choice([0.0, 0.05, 0.2, 0.5]))
        want = oracle_pick(te, ts, es, hist, n_arena, thr)
        got = gpu_pick(te, ts, es, hist, n_arena, thr)
        if want is None:
            assert got[0] == -1, (trial, got)
            arena = [e for e in range(E) if 0 <= es[e] < n_arena]
            assert got[1] == min(arena, key=lambda e: (hist[e], e))
        else:
            assert got == want, (trial, T, E, k, got, want)
            cases += 1
    say(f"hot_pick: {cases} of 60 random tables had a qualifying miss")
    assert cases > 20


def test_hot_pick_grid_stride_many_tokens():
    """More tokens than 256 workgroups x 256 threads: every workgroup walks
    several tokens, and the best miss sits in the last, ragged stretch."""
    rng = np.random.default_rng(5)
    T, E, k = 70001, 64, 4
    te = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    ts = (rng.integers(1, 9, size=(T, k)) / 16.0).astype(np.float32)
    es = np.full(E, -1, dtype=np.int32)
    es[:40] = np.arange(40)
    ts[T - 3, :] = [1.0, 1e-3, 1e-3, 1e-3]
    te[T - 3, :] = [50, 0, 1, 2]          # expert 50 is not resident
    hist = rng.integers(0, 4, size=E).astype(np.float64)
    want = oracle_pick(te, ts, es, hist, 30, 0.2)
    got = gpu_pick(te, ts, es, hist, 30, 0.2)
    assert want is not None and want[0] == 50
    assert got == want, (got, want)


def test_hot_pick_empty_batch():
    got = gpu_pick(np.zeros((0, 4), np.int32), np.zeros((0, 4), np.float32),
                   np.array([0, 1, -1, 2]), np.array([3.0, 1.0, 0.0, 1.0]), 3)
    assert got == [-1, 1]


def test_hot_pick_ring_excluded_decode():
    """Decode workload: ring slots (ids >= 166) are never the eviction choice.
    The kernel is fed the oracle's float32-rounded scores and its history."""
    lay = fixtures.make_layer("decode")
    r = moe.route(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, lay.cfg.k)
    hist = moe.demand(r["topk_expert"], r["topk_score"], lay.cfg.E)
    n_arena = lay.extra["n_resident"]
    got = gpu_pick(r["topk_expert"], r["topk_score"], lay.expert_slot, hist, n_arena, 0.0)
    want = check_hot_pick(got, r["topk_expert"], r["topk_score"], lay.expert_slot, hist,
                          n_arena, 0.0)
    say(f"decode hot pick (threshold 0): gpu {got}, oracle {want}")
    assert 0 <= lay.expert_slot[got[1]] < n_arena


def test_hot_install_applies_only_a_valid_decision():
    """moe_hot_install: e* takes c's arena slot and c leaves the table; any
    other decision (nothing picked, e* already routable, c on a ring slot or
    not resident, e* == c, ids out of range) leaves the table as it was."""
    import torch
    from resident_expert_routing_amd import binding as B
    E, S, n_arena = 12, 8, 6
    # experts 0-5 hold arena slots 0-5, expert 6 and 7 ring slots 6-7, 8-11 none
    es0 = np.array([3, 0, 5, 1, 4, 2, 6, 7, -1, -1, -1, -1], dtype=np.int32)
    cases = [((9, 2), 5), ((8, 1), 0), ((-1, 2), -1), ((9, -1), -1), ((0, 2), -1),
             ((9, 6), -1), ((9, 8), -1), ((9, 9), -1), ((12, 2), -1), ((9, 12), -1)]
    for (e, c), want in cases:
        es = to_dev(es0)
        pick = to_dev(np.array([e, c], dtype=np.int32))
        out = torch.full((1,), 99, dtype=torch.int32, device=es.device)
        assert B.moe_hot_install(pick, es, E, S, n_arena, out) == B.MOE_OK
        assert B.moe_hot_install(pick, es, E, S, n_arena) == B.MOE_OK  # again, no output
        torch.cuda.synchronize()
        want_es = es0.copy()
        if want >= 0:
            want_es[e], want_es[c] = es0[c], -1
        assert int(out.item()) == want, ((e, c), int(out.item()))
        # the second call sees the updated table: e* is no longer a miss
        assert np.array_equal(es.cpu().numpy(), want_es), (e, c)


def test_hot_read_layer_long():
    """Long prefill chunk: the full hot-read call against the oracle."""
    import torch
    from resident_expert_routing_amd import runtime as R
    lay = fixtures.make_layer("long")
    say("long workload: uploading a fresh arena for the hot read")
    g = GpuLayer(lay)
    n_arena = lay.extra["n_resident"]
    es0 = lay.expert_slot.copy()
    hot = R.HotReader(es0, n_arena, g.x.device)
    stream = torch.cuda.current_stream()
    picked = R.layer_step_hot(g.buf, g.x, g.w_router, g.bias, g.expert_slot, g.hist, g.arena,
                              hot, lay.expert_bytes, stream)
    torch.cuda.synchronize()

    # The oracle's decision from its own values: its float64 scores (the share
    # rule rounds them to float32, the stated precision) and its float64
    # history.  A different GPU decision passes only inside the rounding margins.
    r0 = moe.route(g.x_bits, lay.w_router, lay.bias, es0, g.k)
    got_te = g.buf.topk_expert.cpu().numpy()
    got_ts = g.buf.topk_score.cpu().numpy()
    assert np.array_equal(got_te, r0["topk_expert"])
    np.testing.assert_allclose(got_ts, r0["topk_score"], rtol=1e-6, atol=1e-9)
    want_hist = moe.demand_fast(r0["topk_expert"], r0["topk_score"], g.E)
    np.testing.assert_allclose(g.hist.cpu().numpy(), want_hist, rtol=1e-5, atol=0)
    assert picked is not None, "the long workload has a qualifying miss"
    e_star, c = picked[0], picked[1]
    w_e, w_c = check_hot_pick((e_star, c), r0["topk_expert"], r0["topk_score"], es0, want_hist,
                              n_arena)
    assert w_e >= 0, "the oracle finds a qualifying miss too"
    say(f"hot read: load expert {e_star} into the slot of expert {c} (slot {es0[c]}); "
        f"oracle ({w_e}, {w_c})")
    es1 = es0.copy()
    es1[e_star], es1[c] = es0[c], -1
    assert np.array_equal(g.expert_slot.cpu().numpy(), es1)
    assert np.array_equal(hot.es, es1)

    # the slot now holds e*'s packed bytes, verbatim
    slot = int(es1[e_star])
    sb = g.arena.slot_bytes
    got_bytes = g.arena.mem[slot * g.arena.stride: slot * g.arena.stride + sb].cpu().numpy()
    assert np.array_equal(got_bytes, lay.expert_bytes(e_star)[:sb])

    # re-routing over the new routable set and the experts on sampled tokens
    r1 = moe.route(g.x_bits, lay.w_router, lay.bias, es1, g.k)
    _, offsets, perm = moe.bucket(r1["sel_slot"], g.S)
    got = g.routing()
    for key in ("topk_expert", "sel_expert", "sel_slot"):
        assert np.array_equal(got[key], r1[key]), key
    assert np.array_equal(got["slot_offsets"], offsets)
    assert np.array_equal(got["perm"], perm)
    users = np.nonzero((r1["sel_expert"] == e_star).any(axis=1))[0]
    assert users.size > 0, "some token now routes to the loaded expert"
    rng = np.random.default_rng(12)
    tok = np.unique(np.concatenate([users[:8], rng.choice(g.T, 12, replace=False)]))
    sc = lay.slot_content()

    def slot_bytes(s):
        return lay.expert_bytes(e_star) if s == slot else lay.content_bytes(sc[s])

    o, _ = moe.experts_forward(g.x_bits, r1["sel_expert"], r1["sel_weight"], r1["sel_slot"],
                               slot_bytes, g.H, g.I, tokens=tok)
    err = moe.rel_l2(g.out_f64()[tok], o)
    say(f"  hot-read layer rel-L2 {err:.3e} over {tok.size} tokens "
        f"({min(8, users.size)} of them use the loaded expert)")
    assert err <= OUT_REL_L2


def test_hot_read_layer_no_candidate():
    """Nothing qualifies (threshold above every share): plain layer call, no copy."""
    import torch
    from resident_expert_routing_amd import runtime as R
    lay = fixtures.make_layer("tiny")
    g = GpuLayer(lay)
    hot = R.HotReader(lay.expert_slot, lay.S, g.x.device, threshold=1.5)
    picked = R.layer_step_hot(g.buf, g.x, g.w_router, g.bias, g.expert_slot, g.hist, g.arena,
                              hot, lay.expert_bytes)
    torch.cuda.synchronize()
    assert picked is None
    assert np.array_equal(g.expert_slot.cpu().numpy(), lay.expert_slot)
    r = moe.route(g.x_bits, lay.w_router, lay.bias, lay.expert_slot, g.k)
    assert np.array_equal(g.buf.sel_slot.cpu().numpy(), r["sel_slot"])
