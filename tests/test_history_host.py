"""The demand-history planner on the host (CPU): the oracle's boot fill,
forgetting, gainful-swap cut and re-plan cadence against hand-worked cases and
brute force; the C ABI's history file and boot plan against the oracle and an
independent reader of the documented file format."""
import ctypes
import os
import struct

import numpy as np
import pytest

from oracle import plan
from resident_expert_routing_amd import binding as B


# ---------------------------------------------------------------------------
# oracle pins
# ---------------------------------------------------------------------------
def test_boot_fill_hand_worked():
    """Two layers of four experts, k = 1, five slots.

    Layer 0 [4, 0, 2, 2]: ranks e0 0, e2 1, e3 2, e1 3.  Layer 1 [1, 3, 0, 3]:
    ranks e1 0, e3 1, e0 2, e2 3.  Floors: (0,0) and (1,1).  The rest by
    (larger history, rank, layer): (1,3) 3 r1, (0,2) 2 r1, (0,3) 2 r2, (1,0) 1,
    (0,1) 0 r3 / (1,2) 0 r3 ...  Three more slots: (1,3), (0,2), (0,3).
    Slots in (layer, expert) order: (0,0) 0, (0,2) 1, (0,3) 2, (1,1) 3, (1,3) 4.
    """
    hist = np.array([[4.0, 0.0, 2.0, 2.0], [1.0, 3.0, 0.0, 3.0]])
    t = plan.boot_fill(hist, 5, 1)
    assert t.tolist() == [[0, -1, 1, 2], [-1, 3, -1, 4]]
    # k = 2, four slots: each layer's two hottest, in (layer, expert) order
    t = plan.boot_fill(hist, 4, 2)
    assert t.tolist() == [[0, -1, 1, -1], [-1, 2, -1, 3]]
    # the floor wins over hotter pairs of another layer: layer 0 [9, 8, 7, 6] is
    # hotter everywhere than layer 1 [1, 0, 0, 0], yet layer 1 keeps experts 0
    # and 1 (ties at 0 go to the lower id)
    t = plan.boot_fill(np.array([[9.0, 8.0, 7.0, 6.0], [1.0, 0.0, 0.0, 0.0]]), 4, 2)
    assert t.tolist() == [[0, 1, -1, -1], [2, 3, -1, -1]]
    # more slots than pairs: everything resident
    assert (plan.boot_fill(hist, 100, 1) >= 0).all()
    with pytest.raises(ValueError):
        plan.boot_fill(hist, 3, 2)


def test_boot_fill_fresh_history_is_shared_evenly():
    t = plan.boot_fill(np.zeros((4, 8)), 18, 2)
    counts = (t >= 0).sum(axis=1)
    assert counts.tolist() == [5, 5, 4, 4]         # round-robin, lower layers first
    assert (t[:, :4] >= 0).all() and (t[2:, 4] < 0).all()


def brute_boot(hist, n, k):
    """Literal greedy: floors first, then repeatedly the best remaining pair."""
    L, E = hist.shape
    rank = {}
    for l in range(L):
        for r, e in enumerate(sorted(range(E), key=lambda e: (-hist[l, e], e))):
            rank[(l, e)] = r
    chosen = [p for p in rank if rank[p] < min(k, E)]
    while len(chosen) < min(n, L * E):
        best = None
        for l in range(L):
            for e in range(E):
                if (l, e) in chosen:
                    continue
                key = (-hist[l, e], rank[(l, e)], l)
                if best is None or key < best[0]:
                    best = (key, (l, e))
        chosen.append(best[1])
    t = np.full((L, E), -1)
    for s, p in enumerate(sorted(chosen)):
        t[p] = s
    return t


def test_boot_fill_bruteforce():
    rng = np.random.default_rng(4)
    for _ in range(50):
        L, E, k = int(rng.integers(1, 5)), int(rng.integers(1, 9)), int(rng.integers(1, 4))
        hist = rng.integers(0, 4, size=(L, E)).astype(float)
        n = int(rng.integers(L * min(k, E), L * E + 3))
        assert np.array_equal(plan.boot_fill(hist, n, k), brute_boot(hist, n, k))


def test_gainful_swaps_and_decay():
    hist = np.array([[5.0, 1.0, 0.5], [3.0, 2.0, 0.5]])
    ev = [(0, 2), (1, 2), (0, 1)]
    ld = [(0, 0), (1, 1), (1, 0)]
    # 5 > 0.5, 2 > 0.5, 3 > 1 -> all three gain
    assert plan.gainful_swaps(hist, ev, ld) == 3
    ld2 = [(0, 0), (1, 2), (1, 0)]         # 0.5 > 0.5 is no gain: the cut is at one
    assert plan.gainful_swaps(hist, ev, ld2) == 1
    assert np.array_equal(plan.decay(hist, 0.5), hist / 2)
    assert plan.SENSITIVITY_DECAY["low"] == 1.0


def test_replan_points_cadence():
    ev = [("prefill", 0)] + [("token", 0)] * 7 + [("end", 0)] \
        + [("prefill", 1)] + [("token", 1)] * 3 + [("end", 1)] + [("prefill", 2), ("end", 2)]
    # after the prefill (0); tokens at 1..7: every 3 -> after events 3 and 6; the end
    # (8) with one token since; request 1: prefill (9), tokens 10-12 -> 12, end (13)
    # has none since; request 2: prefill (14), end (15) none since
    assert plan.replan_points(ev, 3) == [0, 3, 6, 8, 9, 12, 14]


# ---------------------------------------------------------------------------
# C ABI against the oracle and the documented format
# ---------------------------------------------------------------------------
def test_boot_plan_matches_oracle():
    rng = np.random.default_rng(9)
    for _ in range(40):
        L, E, k = int(rng.integers(1, 6)), int(rng.integers(1, 40)), int(rng.integers(1, 9))
        hist = (rng.integers(0, 5, size=(L, E)) / 4.0).astype(np.float64)
        hist[rng.random((L, E)) < 0.1] = -0.0       # -0 and +0 tie
        n = int(rng.integers(L * min(k, E), L * E + 5))
        out = np.empty((L, E), dtype=np.int32)
        assert B.moe_boot_plan(hist, L, E, k, n, out) == B.MOE_OK
        assert np.array_equal(out, plan.boot_fill(hist, n, k))
    out = np.empty((2, 4), dtype=np.int32)
    assert B.moe_boot_plan(np.zeros((2, 4)), 2, 4, 3, 5, out) == B.MOE_EINVAL   # floor 6 > 5
    bad = np.zeros((2, 4))
    bad[1, 2] = np.nan
    assert B.moe_boot_plan(bad, 2, 4, 1, 5, out) == B.MOE_EINVAL


def fnv1a(data: bytes) -> int:
    h = 0xcbf29ce484222325
    for c in data:
        h ^= c
        h = (h * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def read_history_file(path):
    """The file format as documented, read independently of the library."""
    raw = open(path, "rb").read()
    assert raw[:8] == b"MOEHIST\x01"
    L, E, tokens = struct.unpack_from("<IIQ", raw, 8)
    body = raw[:24 + 8 * L * E]
    (h,) = struct.unpack_from("<Q", raw, len(body))
    assert len(raw) == len(body) + 8 and h == fnv1a(body)
    return np.frombuffer(raw, dtype="<f8", count=L * E, offset=24).reshape(L, E), tokens


def test_history_file_round_trip_and_format(tmp_path):
    rng = np.random.default_rng(2)
    L, E = 5, 12
    hist = rng.random((L, E)) * 100
    hist[0, 0] = 0.0
    hist[1, 3] = 1e-300
    path = str(tmp_path / "hist.bin")
    assert B.moe_history_save(path, hist, L, E, 123456789) == B.MOE_OK
    assert not os.path.exists(path + ".tmp")
    got, tokens = read_history_file(path)
    assert tokens == 123456789 and np.array_equal(got, hist)
    back = np.full((L, E), -1.0)
    tok = ctypes.c_uint64(0)
    assert B.moe_history_load(path, back, L, E, tok) == B.MOE_OK
    assert tok.value == 123456789 and np.array_equal(back, hist)
    # a second save replaces the file whole
    assert B.moe_history_save(path, hist * 2, L, E, 7) == B.MOE_OK
    assert np.array_equal(read_history_file(path)[0], hist * 2)


def test_history_file_errors(tmp_path):
    L, E = 3, 4
    hist = np.arange(L * E, dtype=np.float64).reshape(L, E)
    path = str(tmp_path / "h.bin")
    assert B.moe_history_save(path, hist, L, E, 1) == B.MOE_OK
    out = np.full((L, E), 9.0)
    # another shape
    assert B.moe_history_load(path, np.zeros((4, 4)), 4, 4) == B.MOE_EFORMAT
    # a flipped byte anywhere
    raw = bytearray(open(path, "rb").read())
    for at in (3, 10, 40, len(raw) - 1):
        bad = bytearray(raw)
        bad[at] ^= 0x10
        p2 = str(tmp_path / f"bad{at}.bin")
        open(p2, "wb").write(bytes(bad))
        assert B.moe_history_load(p2, out, L, E) == B.MOE_EFORMAT, at
    # truncated, and one byte too long
    p3 = str(tmp_path / "short.bin")
    open(p3, "wb").write(bytes(raw[:-3]))
    assert B.moe_history_load(p3, out, L, E) == B.MOE_EFORMAT
    open(p3, "wb").write(bytes(raw) + b"\0")
    assert B.moe_history_load(p3, out, L, E) == B.MOE_EFORMAT
    assert (out == 9.0).all()                    # nothing written on a failed load
    assert B.moe_history_load(str(tmp_path / "missing.bin"), out, L, E) == B.MOE_EIO
    neg = hist.copy()
    neg[2, 1] = -1.0
    assert B.moe_history_save(path, neg, L, E, 0) == B.MOE_EINVAL
    assert B.moe_history_save(str(tmp_path / "no_dir" / "h.bin"), hist, L, E, 0) == B.MOE_EIO
    assert B.moe_history_scale(None, 4, 0.5) == B.MOE_EINVAL
    assert B.moe_history_scale(1 << 20, 4, 1.5) == B.MOE_EINVAL
    assert B.moe_history_scale(1 << 20, 4, float("nan")) == B.MOE_EINVAL
