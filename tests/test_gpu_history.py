"""GPU parity of the demand-history planner over a served sequence: a history
learned earlier is saved, loaded at boot, the arena is filled from it, then two
requests are served (prefill chunk, decode steps) with re-plans after each
prefill, every 8 generated tokens and between requests, each preceded by the
history's forgetting; the history is saved at the end and read back.

Every re-plan is checked against the oracle's decision on its own float64
history (tests/decisions.py margins), the slot tables bit-exact, and the last
step's outputs against the oracle.
"""
import ctypes

import numpy as np
import pytest

import fixtures
from decisions import HIST_REL, check_replan, hist_close
from gpu_helpers import say, to_dev
from oracle import moe, plan

pytestmark = pytest.mark.gpu

OUT_REL_L2 = 5e-3
CFG = fixtures.LayerConfig("hist_small", T=2, H=256, E=32, k=4, I=128, resident=64,
                           zipf=True, beta_key="prefill", seed=626, layers=4)
PREFILL_T, EVERY, SENSITIVITY = 64, 8, "high"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import resident_expert_routing_amd  # noqa: F401
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def oracle_demand(model, table, x_bits):
    L, E = model.L, model.cfg.E
    d = np.zeros((L, E))
    for l, lay in enumerate(model.layers):
        r = moe.route(x_bits, lay.w_router, lay.bias, table[l], model.cfg.k)
        d[l] = moe.demand_fast(r["topk_expert"], r["topk_score"], E)
    return d


def oracle_replan(hist, table, n_swap, k):
    ev, ld, _ = plan.replan(hist, table, n_swap, k)
    g = plan.gainful_swaps(hist, ev, ld)
    return g


def test_history_boot_serve_replan_save(tmp_path):
    import torch
    from resident_expert_routing_amd import runtime as R
    model = fixtures.make_arena_model(CFG, distinct_layers=True)
    cfg, L, E, k = model.cfg, model.L, model.cfg.E, model.cfg.k
    model.prepack()
    n_slots = model.S
    dev = torch.device("cuda", 0)

    # a history learned on earlier traffic (the oracle's demand over 3 batches)
    learned = np.zeros((L, E))
    for s in range(3):
        learned += oracle_demand(model, model.expert_slot_table(),
                                 model.tokens(900 + s, T=PREFILL_T))
    path = str(tmp_path / "history.bin")
    from resident_expert_routing_amd import binding as B
    assert B.moe_history_save(path, learned, L, E, 3 * PREFILL_T) == B.MOE_OK

    # boot: load, fill the arena from it
    hist0, seen = R.load_history(path, L, E)
    assert seen == 3 * PREFILL_T and np.array_equal(hist0, learned)
    table = R.boot_table(hist0, k, n_slots)
    assert np.array_equal(table, plan.boot_fill(learned, n_slots, k))
    sa = R.SharedArena(n_slots, cfg.H, cfg.I, table, dev)
    sa.upload(model.pair_bytes)
    sa.hist.copy_(torch.from_numpy(hist0))
    ad = R.AdaptiveArena(sa, k, model.pair_bytes, every=EVERY, sensitivity=SENSITIVITY,
                         tokens_seen=seen)
    factor = R.SENSITIVITY_DECAY[SENSITIVITY]
    ws = [to_dev(l.w_router) for l in model.layers]
    bs = [to_dev(l.bias) for l in model.layers]
    bufs = {T: R.LayerBuffers(T, cfg.H, E, k, cfg.I, n_slots, dev) for T in (PREFILL_T, cfg.T)}
    stream = torch.cuda.current_stream(dev)

    # the oracle's side of the same sequence
    o_hist, o_table = learned.copy(), table.astype(np.int64)
    n_checked = 0
    last = None

    def step(x_bits):
        nonlocal o_hist, last
        T = x_bits.shape[0]
        buf = bufs[T]
        x = to_dev(x_bits.view(np.int16))
        assert np.array_equal(sa.table.cpu().numpy(), o_table)
        outs = []
        for l in range(L):
            R.route(buf, x, ws[l], bs[l], sa.table[l], stream, hist_row=sa.hist[l])
            R.experts(buf, sa.arena.ptr(), sa.arena.stride, stream)
            outs.append(buf.out.clone())
        o_hist = o_hist + oracle_demand(model, o_table, x_bits)
        last = (x_bits, o_table.copy(), outs)

    def replanned(result, reason):
        nonlocal o_hist, o_table, n_checked
        assert result is not None, reason
        ev, ld = result
        o_hist = plan.decay(o_hist, factor)
        got_hist = sa.hist.cpu().numpy()
        np.testing.assert_allclose(got_hist, o_hist, rtol=HIST_REL, atol=0)
        g = oracle_replan(o_hist, o_table, ad.n_swap, k)
        if len(ev) != g:   # the gain cut may move by one only where a gain is within rounding
            i = min(len(ev), g)
            oev, old, _ = plan.replan(o_hist, o_table, max(len(ev), g), k)
            assert abs(len(ev) - g) == 1 and hist_close(o_hist[old[i]], o_hist[oev[i]]), \
                (reason, len(ev), g)
            g = len(ev)
        _, _, onew = check_replan(ev, ld, sa.table_host, o_hist, o_table, g, k)
        o_table = np.asarray(sa.table_host, dtype=np.int64)
        n_checked += 1
        say(f"  re-plan ({reason}): {len(ev)} gainful swaps of at most {ad.n_swap}")

    say(f"history planner: {L} layers, {n_slots} slots, boot from a saved history")
    for req in range(2):
        step(model.tokens(1000 + req, T=PREFILL_T))
        replanned(ad.on_prefill(PREFILL_T, stream), "prefill")
        for i in range(6 if req == 0 else 3):
            step(model.tokens(2000 + 10 * req + i, T=cfg.T))
            r = ad.on_tokens(cfg.T, stream)
            if (i + 1) * cfg.T % EVERY == 0:
                replanned(r, "tokens")
            else:
                assert r is None
        r = ad.on_request_end(stream)
        replanned(r, "between requests")
    assert [x[0] for x in ad.replans] == ["prefill", "tokens", "between requests", "prefill",
                                          "between requests"]

    # the last step's outputs against the oracle, with the tables it used
    x_bits, tab, outs = last
    pairs = {int(tab[l, e]): (l, e) for l in range(L) for e in range(E) if tab[l, e] >= 0}
    for l, lay in enumerate(model.layers):
        r = moe.route(x_bits, lay.w_router, lay.bias, tab[l], k)
        o, _ = moe.experts_forward(x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                                   lambda s: model.pair_bytes(*pairs[s]), cfg.H, cfg.I)
        bits = outs[l].cpu().numpy().view(np.uint16)
        got = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert moe.rel_l2(got, o) <= OUT_REL_L2, l

    # persisted, and read back bit for bit
    out_path = str(tmp_path / "history2.bin")
    ad.save(out_path, stream)
    back, seen2 = R.load_history(out_path, L, E)
    assert np.array_equal(back, sa.hist.cpu().numpy())
    assert seen2 == seen + 2 * PREFILL_T + 9 * cfg.T
    np.testing.assert_allclose(back, o_hist, rtol=HIST_REL, atol=0)
    say(f"  {n_checked} re-plans checked; history saved and reloaded bit for bit")
