"""The pins are strong enough: plant plausible mistakes in the oracle (on the CPU,
via monkeypatch) and check that a pin fails for each one."""
import numpy as np
import pytest

from oracle import moe, mxfp4
import test_oracle_ffn as tf
import test_oracle_mxfp4 as tm
import test_oracle_routing as tr


def _fails(check):
    with pytest.raises(AssertionError):
        check()


def test_wrong_e2m1_value(monkeypatch):
    bad = mxfp4.VALUE.copy()
    bad[5] = 2.5
    monkeypatch.setattr(mxfp4, "VALUE", bad)
    _fails(tm.check_decode_exhaustive)


def test_wrong_scale_bias(monkeypatch):
    orig = mxfp4.decode

    def dec(p, s):
        return orig(p, np.minimum(np.asarray(s, dtype=np.int64) + 1, 254).astype(np.uint8))
    monkeypatch.setattr(mxfp4, "decode", dec)
    _fails(tm.check_decode_exhaustive)


def test_wrong_tie_rule(monkeypatch):
    monkeypatch.setattr(mxfp4, "_MANT_ODD", 1 - mxfp4._MANT_ODD)
    _fails(tm.check_encode_golden)
    _fails(tm.check_bf16_window)


def test_wrong_scale_exponent(monkeypatch):
    orig = np.frexp

    class NP:  # frexp off by one inside the encoder only
        def __getattr__(self, k):
            return getattr(np, k)

        @staticmethod
        def frexp(a):
            m, e = orig(a)
            return m, e + 1
    monkeypatch.setattr(mxfp4, "np", NP())
    _fails(tm.check_roundtrip)


def test_dropped_bias(monkeypatch):
    orig = moe.router_logits
    monkeypatch.setattr(moe, "router_logits", lambda x, w, b=None: orig(x, w, None))
    _fails(tr.check_logits_fsum)


def test_reversed_ties(monkeypatch):
    def bad(z_row, allowed=None):
        ids = np.arange(z_row.shape[0]) if allowed is None else np.flatnonzero(allowed)
        order = np.argsort(-z_row[ids][::-1], kind="stable")[::-1][::-1]
        return ids[::-1][order]
    monkeypatch.setattr(moe, "rank_order", bad)
    _fails(tr.check_topk_bruteforce)


def test_missing_renormalisation(monkeypatch):
    monkeypatch.setattr(moe, "renormalise", lambda p, picks: moe.gather(p, picks))
    _fails(tr.check_softmax_and_renorm)


def test_demand_skips_a_pick(monkeypatch):
    orig = moe.demand
    monkeypatch.setattr(moe, "demand", lambda te, ts, E: orig(te[:, 1:], ts[:, 1:], E))
    _fails(tr.check_demand)


def test_unstable_bucket(monkeypatch):
    def bad(sel_slot, S):
        c, o, p = orig(sel_slot, S)
        for s in range(S):
            p[o[s]:o[s + 1]] = p[o[s]:o[s + 1]][::-1]
        return c, o, p
    orig = moe.bucket
    monkeypatch.setattr(moe, "bucket", bad)
    _fails(tr.check_bucket)


def test_wrong_silu_sign(monkeypatch):
    monkeypatch.setattr(moe, "silu", lambda v: v / (1.0 + np.exp(v)))
    _fails(tf.check_ffn_bruteforce)


def test_gate_up_swapped(monkeypatch):
    orig = moe.expert_ffn
    monkeypatch.setattr(moe, "expert_ffn", lambda x, W, act="mxfp4": orig(x, (W[1], W[0], W[2]), act))
    _fails(tf.check_ffn_bruteforce)


def test_combine_drops_last_pick(monkeypatch):
    orig = moe.combine
    monkeypatch.setattr(moe, "combine", lambda y, w, se: orig(y[:, :-1], w[:, :-1], se[:, :-1]))
    _fails(tf.check_identical_experts)


def test_shared_expert_weighted_or_dropped(monkeypatch):
    monkeypatch.setattr(moe, "shared_combine", lambda out, ys: out + 0.5 * ys)
    _fails(tf.test_shared_expert_closed_forms)
    monkeypatch.setattr(moe, "shared_combine", lambda out, ys: out)
    _fails(tf.test_shared_expert_closed_forms)


def test_ring_plan_ignores_pending(monkeypatch):
    """A ring plan that forgets the pairs already in flight picks one twice."""
    import test_oracle_plan as tp
    from oracle import plan
    orig = plan.ring_plan
    monkeypatch.setattr(plan, "ring_plan",
                        lambda w, t, ring, head, per, s0: orig(w, t, [-1] * len(ring), head,
                                                               per, s0))
    _fails(tp.test_ring_pending_pairs_not_planned_twice_and_stale_install_skipped)


def test_boot_fill_without_floor(monkeypatch):
    import test_history_host as th
    from oracle import plan
    orig = plan.boot_fill
    monkeypatch.setattr(plan, "boot_fill", lambda h, n, k: orig(h, n, 0))
    _fails(th.test_boot_fill_hand_worked)


# ---- MXFP6 (E2M3) ----
import test_oracle_mxfp6 as t6  # noqa: E402
from oracle import mxfp6  # noqa: E402


def test_mxfp6_wrong_value(monkeypatch):
    bad = mxfp6.VALUE.copy()
    bad[19] = 2.625
    monkeypatch.setattr(mxfp6, "VALUE", bad)
    _fails(t6.test_decode_exhaustive)


def test_mxfp6_wrong_tie_rule(monkeypatch):
    monkeypatch.setattr(mxfp6, "_MANT_ODD", 1 - mxfp6._MANT_ODD)
    _fails(t6.test_ties_to_even_mantissa_and_scale)
    _fails(t6.test_bf16_window_exact_rounding)


def test_mxfp6_element_bits_swapped(monkeypatch):
    orig = mxfp6.pack

    def pack(codes):   # the two 3-bit halves of every code exchanged
        c = np.asarray(codes, dtype=np.uint8)
        return orig(((c & 7) << 3) | (c >> 3))
    monkeypatch.setattr(mxfp6, "pack", pack)
    _fails(t6.test_packing_hand_worked)


def test_mxfp6_scale_from_fp4_exponent(monkeypatch):
    orig = np.frexp

    class NP:  # the block exponent one too large (as if the element maximum were 2^3)
        def __getattr__(self, k):
            return getattr(np, k)

        @staticmethod
        def frexp(a):
            m, e = orig(a)
            return m, e + 1
    monkeypatch.setattr(mxfp6, "np", NP())
    _fails(t6.test_round_trip_every_value_at_many_scales)


def test_slot_codes_read_row_major(monkeypatch):
    # the oracle reading code bytes row by row instead of in 16-row tiles
    monkeypatch.setattr(moe, "code_position", lambda n, j, nb: n * nb + j)
    _fails(tf.test_slot_code_tiles_hand_worked)


def test_slot_tiles_unit_major(monkeypatch):
    # inside a tile, the 16-byte units of all 16 rows first, then the next unit
    def pos(n, j, nb):
        c = j // 64
        return (n // 16) * (16 * nb) + c * 1024 + ((j - 64 * c) // 16) * 256 + (n % 16) * 16 \
            + j % 16
    monkeypatch.setattr(moe, "code_position", pos)
    _fails(tf.test_slot_code_tiles_hand_worked)
