"""Seeded workload generators: determinism, residency counts, Zipf calibration."""
import math

import numpy as np
import pytest

import fixtures
from oracle import moe, plan


def test_seeds_reproduce_bytes():
    a = fixtures.make_layer("tiny")
    b = fixtures.make_layer("tiny")
    assert np.array_equal(a.x_bits, b.x_bits)
    assert np.array_equal(a.w_router, b.w_router)
    assert np.array_equal(a.expert_slot, b.expert_slot)
    assert np.array_equal(a.expert_bytes(3), b.expert_bytes(3))
    c = fixtures.make_layer("tiny", x_stream=1)
    assert not np.array_equal(a.x_bits, c.x_bits)


@pytest.mark.parametrize("name,res,ring", [("tiny", 10, 0), ("decode", 166, 64),
                                           ("prefill", 166, 0), ("long", 130, 0)])
def test_residency_counts(name, res, ring):
    lay = fixtures.make_layer(name, T=4)
    assert lay.S == res + ring
    assert (lay.expert_slot >= 0).sum() == res + ring
    assert sorted(lay.expert_slot[lay.expert_slot >= 0]) == list(range(res + ring))
    assert np.array_equal(lay.expert_slot[lay.slot_expert], np.arange(lay.S))


def test_decode_and_prefill_share_the_model():
    d = fixtures.make_layer("decode", T=4)
    p = fixtures.make_layer("prefill", T=4)
    assert np.array_equal(d.w_router, p.w_router) and np.array_equal(d.bias, p.bias)
    assert np.array_equal(d.slot_expert[:166], p.slot_expert)


def test_slot_layout_sizes():
    assert fixtures.SlotLayout(256, 128).nbytes == 52224
    assert fixtures.SlotLayout(4096, 2048).nbytes == 13369344
    assert fixtures.SlotLayout(6144, 2048).nbytes == 20054016
    sec = moe.slot_sections(4096, 2048)
    assert sec["total"] == 13369344
    for name, (off, sz) in fixtures.SlotLayout(4096, 2048).sections.items():
        assert off % 256 == 0 and sec[name][0] == off


def test_zipf_calibration_holds():
    lay = fixtures.make_layer("prefill")
    z = moe.router_logits(lay.x_bits, lay.w_router, lay.bias)
    picks = moe.topk(z, 8)
    counts = np.sort(np.bincount(picks.reshape(-1), minlength=256))[::-1]
    share = counts[:math.ceil(0.1 * 256)].sum() / picks.size
    assert abs(share - 0.5) <= 0.01, share


def test_arena40_counts():
    c = fixtures.arena40_layer_counts()
    assert c.sum() == 6666 and c.min() >= 103 and c.max() <= 230 and len(c) == 40


@pytest.mark.slow
def test_long_workload_has_a_hot_miss():
    lay = fixtures.make_layer("long")
    r = moe.route(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, 8)
    d = moe.demand_fast(r["topk_expert"], r["topk_score"], 192)
    got = plan.hot_read(r["topk_score"], r["topk_expert"], lay.expert_slot, d, n_arena=130)
    assert got is not None
