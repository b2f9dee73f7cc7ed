"""GPU parity of the asynchronous hot ring over a multi-step run: a 4-layer
shared arena with an 8-entry ring on top, 3 picks a step, 12 steps driven by
runtime.HotRing exactly as a serving loop would (plan on the device after each
step, copies on a side stream while the next step runs, install before the
step after).  Every step's slot tables, ring picks and every layer's output
are checked against the oracle's simulation of the same loop.

Bars: tables bit-exact at every step; picks equal to the oracle's ring_plan
on its own float64 step demand, or different only inside the demand margin
(tests/decisions.py); ring slots hold their pairs' bytes verbatim; routing
bit-exact; output relative L2 <= 5e-3.
"""
import numpy as np
import pytest

import fixtures
from decisions import check_ring_plan
from gpu_helpers import say, to_dev
from oracle import moe, plan

pytestmark = pytest.mark.gpu

OUT_REL_L2 = 5e-3

SMALL = fixtures.LayerConfig("ring_small", T=16, H=256, E=32, k=4, I=128, resident=64,
                             zipf=True, beta_key="prefill", seed=616, layers=4)
R, PER_STEP, STEPS = 8, 3, 12


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import resident_expert_routing_amd  # noqa: F401
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def slot_pairs(table, S):
    out = {}
    l, e = np.nonzero(table >= 0)
    for li, ei in zip(l, e):
        out[int(table[li, ei])] = (int(li), int(ei))
    return out


def test_hot_ring_multi_step():
    import torch
    from resident_expert_routing_amd import runtime as R_
    model = fixtures.make_arena_model(SMALL, distinct_layers=True)
    cfg, L, E = model.cfg, model.L, model.cfg.E
    model.prepack()
    n_arena = model.S
    S = n_arena + R
    table0 = model.expert_slot_table()
    dev = torch.device("cuda", 0)
    sa = R_.SharedArena(S, cfg.H, cfg.I, table0, dev)
    sa.upload(model.pair_bytes)
    ring = R_.HotRing(sa, n_arena, R, PER_STEP, model.pair_bytes, dev, keep_picks=True)
    buf = R_.LayerBuffers(cfg.T, cfg.H, E, cfg.k, cfg.I, S, dev)
    stream = torch.cuda.current_stream(dev)
    ws = [to_dev(l.w_router) for l in model.layers]
    bs = [to_dev(l.bias) for l in model.layers]
    xs = [to_dev(model.tokens(s).view(np.int16)) for s in range(STEPS)]
    snaps, outs = [], []
    say(f"hot ring: {L} layers, {n_arena} arena slots + {R} ring entries, {PER_STEP} picks a "
        f"step, {STEPS} steps")
    for s in range(STEPS):
        ring.before_step(s, stream)
        snaps.append(sa.table.clone())             # the tables this step routes with
        step_out = []
        for l in range(L):
            R_.route(buf, xs[s], ws[l], bs[l], sa.table[l], stream, hist_row=sa.hist[l],
                     delta=ring.delta_row(l))
            R_.experts(buf, sa.arena.ptr(), sa.arena.stride, stream)
            step_out.append(buf.out.clone())
        outs.append(step_out)
        ring.after_step(s, stream)
    ring.finish(STEPS - 1)
    torch.cuda.synchronize()

    # the oracle's simulation of the same loop
    tab = table0.copy()
    oring, head = [-1] * R, 0
    plans = {}
    n_picked = n_routed_ring = 0
    worst = 0.0
    for s in range(STEPS):
        if s >= 2:
            tab = plan.ring_install(plans[s - 2], tab, oring, n_arena)
        got_tab = snaps[s].cpu().numpy()
        assert np.array_equal(got_tab, tab), f"step {s}: slot tables differ"
        pairs = slot_pairs(tab, S)
        weight = np.zeros((L, E))
        x_bits = model.tokens(s)
        for l, lay in enumerate(model.layers):
            r = moe.route(x_bits, lay.w_router, lay.bias, tab[l], cfg.k)
            weight[l] = moe.demand_fast(r["topk_expert"], r["topk_score"], E)
            n_routed_ring += int((r["sel_slot"] >= n_arena).sum())
            o, _ = moe.experts_forward(x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                                       lambda sl: model.pair_bytes(*pairs[sl]), cfg.H, cfg.I)
            bits = outs[s][l].cpu().numpy().view(np.uint16)
            got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            err = moe.rel_l2(got, o)
            assert err <= OUT_REL_L2, (s, l, err)
            worst = max(worst, err)
        p, tab, oring, head = check_ring_plan(ring.picks[s], weight, tab, oring, head,
                                              PER_STEP, n_arena)
        plans[s] = p
        n_picked += len(p)
    assert np.array_equal(ring.ring.cpu().numpy()[1:], np.array(oring))
    # every ring entry's bytes are those of the pair its last copy loaded
    torch.cuda.synchronize()
    a = sa.arena
    for rr, pid in enumerate(oring):
        if pid < 0:
            continue
        s0 = (n_arena + rr) * a.stride
        got_b = a.mem[s0: s0 + a.slot_bytes].cpu().numpy()
        assert np.array_equal(got_b, model.pair_bytes(pid // E, pid % E)), (rr, pid)
    say(f"  {n_picked} ring picks over {STEPS} steps, {n_routed_ring} routed assignments served "
        f"from ring slots; tables bit-exact every step; worst rel-L2 {worst:.3e}")
    assert n_picked >= PER_STEP * (STEPS - 1)        # the ring kept filling
    assert n_routed_ring > 0                          # and the filled entries were used


def test_ring_plan_kernel_random_tables():
    """moe_ring_plan alone on random tables, weights with ties, wrap-around and
    pairs already in the ring, against the oracle (same float32 weights)."""
    import torch
    from resident_expert_routing_amd import binding as B
    rng = np.random.default_rng(21)
    for trial in range(40):
        L, E = int(rng.integers(1, 41)), int(rng.integers(2, 257))
        if L * E > B.MOE_MAX_RING_PAIRS:
            E = B.MOE_MAX_RING_PAIRS // L
        Rr = int(rng.integers(1, 65))
        per = int(rng.integers(1, min(Rr, 64) + 1))
        slot0 = 1000
        table = np.where(rng.random((L, E)) < 0.5, 7, -1).astype(np.int32)
        w = (rng.integers(0, 5, size=(L, E)) / 8.0).astype(np.float32)
        ring_state = np.full(Rr, -1, dtype=np.int64)
        fill = rng.choice(L * E, size=min(Rr, L * E) // 2, replace=False)
        ring_state[:fill.size] = fill
        for r, pid in enumerate(ring_state):     # some ring pairs are installed
            if pid >= 0 and rng.random() < 0.5:
                table[pid // E, pid % E] = slot0 + r
        head = int(rng.integers(0, Rr))
        want = plan.ring_plan(w, table, ring_state, head, per, slot0)
        t_dev = to_dev(table)
        ring_dev = to_dev(np.concatenate([[head], ring_state]).astype(np.int32))
        plan_dev = torch.full((1 + 3 * per,), -7, dtype=torch.int32, device="cuda")
        B.check(B.moe_ring_plan(to_dev(w), t_dev, L, E, ring_dev, Rr, slot0, per, plan_dev),
                "moe_ring_plan")
        torch.cuda.synchronize()
        pl = plan_dev.cpu().numpy()
        got = [tuple(int(v) for v in pl[1 + 3 * i: 4 + 3 * i]) for i in range(pl[0])]
        assert got == [tuple(p) for p in want[0]], (trial, got, want[0])
        assert np.array_equal(t_dev.cpu().numpy(), want[1]), trial
        rd = ring_dev.cpu().numpy()
        assert rd[0] == want[3] and np.array_equal(rd[1:], want[2]), trial
        # the install makes exactly the plan's pairs routable
        B.check(B.moe_ring_install(plan_dev, t_dev, L, E, ring_dev, Rr, slot0),
                "moe_ring_install")
        torch.cuda.synchronize()
        assert np.array_equal(t_dev.cpu().numpy(),
                              plan.ring_install(want[0], want[1], want[2], slot0)), trial
