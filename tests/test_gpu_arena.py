"""GPU parity of the shared arena and its re-plan: several layers route and
accumulate demand into one [L][E] history, the re-plan (moe_replan) swaps the
coldest resident pairs for the hottest missing ones, the copies land in the
right slots, and the next step's routing and outputs match the oracle run with
the new tables.

Bars: demand history within 1e-5 relative of the oracle's sums over steps;
swap lists and tables bit-exact against the oracle's re-plan on the device's
history; slot bytes verbatim; routing bit-exact; output relative L2 <= 5e-3.
"""
import numpy as np
import pytest

import fixtures
from oracle import moe, plan
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


def check_step(model, table, res, step, pair_of_slot):
    x_bits = model.tokens(step)
    cfg = model.cfg
    for l, lay in enumerate(model.layers):
        r = moe.route(x_bits, lay.w_router, lay.bias, table[l], cfg.k)
        _, offsets, perm = moe.bucket(r["sel_slot"], model.S)
        got, out = res[l]
        for key in ("topk_expert", "sel_expert", "sel_slot"):
            assert np.array_equal(got[key], r[key]), (l, key)
        assert np.array_equal(got["slot_offsets"], offsets) and np.array_equal(got["perm"], perm)
        o, _ = moe.experts_forward(x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                                   lambda s: model.pair_bytes(*pair_of_slot[s]), cfg.H, cfg.I)
        err = moe.rel_l2(out, o)
        assert err <= OUT_REL_L2, (l, err)


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
    want_hist = np.zeros((L, cfg.E))
    for step in range(steps):
        res = run_step(model, sa, buf, step)
        if step == 0:
            check_step(model, table0, res, step, model.slot_pairs(table0))
        for l, lay in enumerate(model.layers):
            r = moe.route(model.tokens(step), lay.w_router, lay.bias, table0[l], cfg.k)
            want_hist[l] += moe.demand_fast(r["topk_expert"], r["topk_score"], cfg.E)
    hist = sa.hist.cpu().numpy()
    np.testing.assert_allclose(hist, want_hist, rtol=1e-5, atol=0)
    assert np.array_equal(hist == 0, want_hist == 0)

    n_swap = 8
    ev, ld = sa.replan(cfg.k, n_swap, model.pair_bytes)
    torch.cuda.synchronize()
    oev, old, onew = plan.replan(hist, table0, n_swap, cfg.k)
    m = min(len(oev), len(old))
    say(f"re-plan: evict {ev}, load {ld}")
    assert len(ev) == m == n_swap
    assert ev == [tuple(map(int, p)) for p in oev[:m]]
    assert ld == [tuple(map(int, p)) for p in old[:m]]
    assert np.array_equal(sa.table_host, onew)
    assert np.array_equal(sa.table.cpu().numpy(), onew)
    # a busy layer can gain slots while a quiet one gives them up
    moved = sum(1 for (le, _), (ll, _) in zip(ev, ld) if le != ll)
    say(f"  {moved} of {m} swaps move a slot between layers")

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
