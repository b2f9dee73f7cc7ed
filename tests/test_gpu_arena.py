"""GPU parity of the shared arena and its re-plan: several layers route and
accumulate demand into one [L][E] history, the re-plan (moe_replan) swaps the
coldest resident pairs for the hottest missing ones, the copies land in the
right slots, and the next step's routing and outputs match the oracle run with
the new tables.

Bars: demand history within 1e-5 relative of the oracle's sums over steps;
swap lists and tables equal to the oracle's re-plan on the oracle's own
float64 history, or different only where the oracle's history values are
within that 1e-5 margin (tests/decisions.py); slot bytes verbatim; routing
bit-exact; output relative L2 <= 5e-3.
"""
import numpy as np
import pytest

import fixtures
from oracle import moe
from decisions import check_replan
from gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu

OUT_REL_L2 = 5e-3

SMALL = fixtures.LayerConfig("arena_small", T=16, H=256, E=32, k=4, I=128, resident=64,
                             zipf=True, beta_key="prefill", seed=606, layers=4)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import resident_expert_routing_amd  # noqa: F401
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def run_step(model, sa, buf, step, with_demand=True):
    """All layers on one step's tokens; returns per-layer (routing, out) on the host."""
    import torch
    from resident_expert_routing_amd import runtime as R
    cfg = model.cfg
    x = to_dev(model.tokens(step).view(np.int16))
    res = []
    for l, lay in enumerate(model.layers):
        R.route(buf, x, to_dev(lay.w_router), to_dev(lay.bias), sa.table[l],
                hist_row=sa.hist[l] if with_demand else None)
        R.experts(buf, sa.arena.ptr(), sa.arena.stride)
        torch.cuda.synchronize()
        bits = buf.out.cpu().numpy().view(np.uint16)
        out = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        res.append(({"topk_expert": buf.topk_expert.cpu().numpy(),
                     "sel_expert": buf.sel_expert.cpu().numpy(),
                     "sel_slot": buf.sel_slot.cpu().numpy(),
                     "slot_offsets": buf.slot_offsets.cpu().numpy(),
                     "perm": buf.perm.cpu().numpy()}, out))
    return res


def check_step(model, table, res, step, pair_of_slot, decoded=None):
    x_bits = model.tokens(step)
    cfg = model.cfg
    worst = 0.0
    for l, lay in enumerate(model.layers):
        r = moe.route(x_bits, lay.w_router, lay.bias, table[l], cfg.k)
        _, offsets, perm = moe.bucket(r["sel_slot"], model.S)
        got, out = res[l]
        for key in ("topk_expert", "sel_expert", "sel_slot"):
            assert np.array_equal(got[key], r[key]), (l, key)
        assert np.array_equal(got["slot_offsets"], offsets) and np.array_equal(got["perm"], perm)
        o, _ = moe.experts_forward(x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                                   lambda s: model.pair_bytes(*pair_of_slot[s]), cfg.H, cfg.I,
                                   decoded=decoded)
        err = moe.rel_l2(out, o)
        assert err <= OUT_REL_L2, (l, err)
        worst = max(worst, err)
    return worst


def oracle_history(model, table, steps):
    """The oracle's float64 [L][E] demand history over the given steps."""
    cfg = model.cfg
    hist = np.zeros((model.L, cfg.E))
    for step in steps:
        x_bits = model.tokens(step)
        for l, lay in enumerate(model.layers):
            r = moe.route(x_bits, lay.w_router, lay.bias, table[l], cfg.k)
            hist[l] += moe.demand_fast(r["topk_expert"], r["topk_score"], cfg.E)
    return hist


def test_shared_arena_replan_small():
    import torch
    from resident_expert_routing_amd import runtime as R
    model = fixtures.make_arena_model(SMALL, distinct_layers=True)
    cfg, L = model.cfg, model.L
    model.prepack()
    table0 = model.expert_slot_table()
    say(f"shared arena: {L} layers, {model.S} slots, counts {model.counts.tolist()}")
    dev = torch.device("cuda", 0)
    sa = R.SharedArena(model.S, cfg.H, cfg.I, table0, dev)
    sa.upload(model.pair_bytes)
    buf = R.LayerBuffers(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, model.S, dev)

    steps = 6
    for step in range(steps):
        res = run_step(model, sa, buf, step)
        if step == 0:
            check_step(model, table0, res, step, model.slot_pairs(table0))
    want_hist = oracle_history(model, table0, range(steps))
    hist = sa.hist.cpu().numpy()
    np.testing.assert_allclose(hist, want_hist, rtol=1e-5, atol=0)
    assert np.array_equal(hist == 0, want_hist == 0)

    n_swap = 8
    ev, ld = sa.replan(cfg.k, n_swap, model.pair_bytes)
    torch.cuda.synchronize()
    say(f"re-plan: evict {ev}, load {ld}")
    assert len(ev) == n_swap
    onew = sa.table_host
    check_replan(ev, ld, onew, want_hist, table0, n_swap, cfg.k)
    assert np.array_equal(sa.table.cpu().numpy(), onew)
    # a busy layer can gain slots while a quiet one gives them up
    moved = sum(1 for (le, _), (ll, _) in zip(ev, ld) if le != ll)
    say(f"  {moved} of {n_swap} swaps move a slot between layers")

    pairs = model.slot_pairs(onew)
    a = sa.arena
    for (ll, el) in ld:
        s = int(onew[ll, el])
        got = a.mem[s * a.stride: s * a.stride + a.slot_bytes].cpu().numpy()
        assert np.array_equal(got, model.pair_bytes(ll, el)), (ll, el, s)

    res = run_step(model, sa, buf, steps, with_demand=False)
    check_step(model, onew, res, steps, pairs)


def test_shared_arena_replan_nothing_to_swap():
    import torch
    from resident_expert_routing_amd import runtime as R
    cfg = fixtures.LayerConfig("arena_tiny", T=4, H=256, E=8, k=4, I=128, resident=8, seed=607,
                               layers=2)
    model = fixtures.make_arena_model(cfg)
    table0 = model.expert_slot_table()
    sa = R.SharedArena(model.S, cfg.H, cfg.I, table0, torch.device("cuda", 0))
    # every layer sits at its floor (4 residents each, k = 4): nothing can move
    assert (model.counts == 4).all()
    ev, ld = sa.replan(cfg.k, 3, model.pair_bytes)
    assert ev == [] and ld == []
    assert np.array_equal(sa.table.cpu().numpy(), table0)


@pytest.mark.timeout(900)
def test_shared_arena_replan_arena40():
    """The 40-layer shared arena at its real shape: 40 x 256 experts, hidden
    4096, intermediate 2048, 6666 slots (89 GB), 32 tokens a layer call.
    Three steps of demand, the 5 % re-plan (333 swaps, moe_replan's prebuilt
    work lists past 1024 slots), then every layer of the next step against the
    oracle run with the new tables."""
    import torch
    from resident_expert_routing_amd import runtime as R
    model = fixtures.make_arena_model("arena40")
    cfg, L = model.cfg, model.L
    say(f"arena40: {L} layers, {model.S} slots; packing {cfg.n_contents} expert contents")
    model.prepack()
    table0 = model.expert_slot_table()
    dev = torch.device("cuda", 0)
    sa = R.SharedArena(model.S, cfg.H, cfg.I, table0, dev)
    sa.upload(model.pair_bytes)
    buf = R.LayerBuffers(cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, model.S, dev)
    decoded = {}
    steps = 3
    for step in range(steps):
        say(f"  arena40 step {step}: {L} layer calls")
        res = run_step(model, sa, buf, step)
        if step == 0:
            err = check_step(model, table0, res, step, model.slot_pairs(table0), decoded)
            say(f"  step 0: every layer bit-exact routing, worst rel-L2 {err:.3e}")
    want_hist = oracle_history(model, table0, range(steps))
    hist = sa.hist.cpu().numpy()
    np.testing.assert_allclose(hist, want_hist, rtol=1e-5, atol=0)
    assert np.array_equal(hist == 0, want_hist == 0)

    n_swap = model.S // 20
    assert n_swap == 333
    ev, ld = sa.replan(cfg.k, n_swap, model.pair_bytes)
    torch.cuda.synchronize()
    onew = sa.table_host
    check_replan(ev, ld, onew, want_hist, table0, n_swap, cfg.k)
    assert np.array_equal(sa.table.cpu().numpy(), onew)
    moved = sum(1 for (le, _), (ll, _) in zip(ev, ld) if le != ll)
    say(f"  re-plan: {len(ev)} swaps, {moved} move a slot between layers")
    a = sa.arena
    for (ll, el) in ld:
        s = int(onew[ll, el])
        got = a.mem[s * a.stride: s * a.stride + a.slot_bytes].cpu().numpy()
        assert np.array_equal(got, model.pair_bytes(ll, el)), (ll, el, s)
    res = run_step(model, sa, buf, steps, with_demand=False)
    err = check_step(model, onew, res, steps, model.slot_pairs(onew), decoded)
    say(f"  step after the re-plan: every layer bit-exact routing, worst rel-L2 {err:.3e}")
