"""GPU parity of the MXFP6 activation variant (act_format = MOE_ACT_MXFP6):
activation rows and the experts' h rows in MXFP6 (E2M3 elements, E8M0 scale
per 32), weights MXFP4 as in the pages' layer (TideLM README, expert format;
the activation format is this library's reading, the OCP MX v1.0 FP6 E2M3
element).  The HIP path through the C ABI against the oracle run with
act='mxfp6', on both kernel families (small batches; the pipelined kernels
from 2048 assignments).

Bars: routing outputs as in the MXFP4 runs (the format changes no pick);
activation bytes bit-exact against the oracle's MXFP6 encoder; layer output
relative L2 <= 5e-3 pooled, every token <= 5e-2, at most 0.5 % of tokens
above 5e-3 (the layer parity bars: a flipped E2M3 rounding edge in h moves a
y row by at most one code step, a quarter of an E2M1 step).
"""
import numpy as np
import pytest

import fixtures
from gpu_helpers import GpuLayer, say, to_dev
from oracle import moe, mxfp6

pytestmark = pytest.mark.gpu

FP6 = 1  # MOE_ACT_MXFP6
OUT_REL_L2 = 5e-3
TOKEN_REL_L2_MAX = 5e-2
TOKEN_OVER_BAR_FRAC = 5e-3


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import resident_expert_routing_amd  # noqa: F401
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def oracle_route(g):
    r = moe.route(g.x_bits, g.lay.w_router, g.lay.bias, g.expert_slot_np, g.k)
    _, offsets, perm = moe.bucket(r["sel_slot"], g.S)
    r["slot_offsets"], r["perm"] = offsets, perm
    return r


def check_route_fp6(g, r):
    got = g.routing()
    for key in ("topk_expert", "sel_expert", "sel_slot", "slot_offsets", "perm"):
        assert np.array_equal(got[key], r[key]), key
    np.testing.assert_allclose(got["sel_weight"], r["sel_weight"], rtol=0, atol=1e-6)
    H = g.H
    if g.T:
        codes, scales = mxfp6.encode(moe.bf16_to_f64(g.x_bits))
        assert got["xq"].shape[1] == (3 * H // 4 + H // 32 + 15) // 16 * 16
        assert np.array_equal(got["xq"][:, :3 * H // 4], codes), "xq codes"
        assert np.array_equal(got["xq"][:, 3 * H // 4:3 * H // 4 + H // 32], scales), "xq scales"


def layer_check(g, tokens=None, shared=None):
    from resident_expert_routing_amd import runtime as R
    g.route()
    R.experts(g.buf, g.arena.ptr(), g.arena.stride,
              shared_expert=None if shared is None else to_dev(shared))
    out = g.out_f64()
    r = oracle_route(g)
    check_route_fp6(g, r)
    o, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                               g.slot_bytes_fn(), g.H, g.I, act="mxfp6", tokens=tokens,
                               shared_bytes=shared)
    got = out if tokens is None else out[tokens]
    err = moe.rel_l2(got, o)
    per = np.linalg.norm(got - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-300)
    over = int((per > OUT_REL_L2).sum())
    say(f"  rel-L2 {err:.3e} over {got.shape[0]} tokens, max per token {per.max():.3e}, "
        f"{over} above {OUT_REL_L2}")
    assert err <= OUT_REL_L2, err
    assert per.max() <= TOKEN_REL_L2_MAX, (per.max(), int(per.argmax()))
    assert over <= TOKEN_OVER_BAR_FRAC * got.shape[0], over
    return err, out


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_mxfp6_route_bytes(name):
    """Both encoders (the router-side one of small batches, the selection-side
    one of larger batches) against the oracle's MXFP6 encoder."""
    lay = fixtures.make_layer(name)
    say(f"MXFP6 activation rows, workload {name}")
    g = GpuLayer(lay, act_format=FP6)
    g.route()
    check_route_fp6(g, oracle_route(g))


@pytest.mark.parametrize("name", ["small", "decode"])
def test_mxfp6_layer_parity(name):
    say(f"MXFP6 layer parity {name} (every token)")
    if name == "small":  # the tiny workload's counts at the smallest supported H, I
        lay = fixtures.tiny_layer(T=64, H=512, E=16, k=4, I=512, n_routable=10, seed=101)
    else:
        lay = fixtures.make_layer(name)
    layer_check(GpuLayer(lay, act_format=FP6))


@pytest.mark.timeout(600)
def test_mxfp6_layer_parity_prefill_all_tokens():
    """2048 tokens (16384 assignments) on the pipelined kernels: every token
    (every M-tile and N-tile of every slot)."""
    g = GpuLayer(fixtures.make_layer("prefill"), act_format=FP6)
    say(f"MXFP6 layer parity prefill, all {g.T} tokens")
    layer_check(g)


@pytest.mark.timeout(900)
def test_mxfp6_layer_parity_long_sampled():
    """8192 tokens, H = 6144 (65536 assignments, slots of up to ~4800 rows);
    256 tokens sampled for the oracle."""
    g = GpuLayer(fixtures.make_layer("long"), act_format=FP6)
    tokens = np.sort(np.random.default_rng(8).choice(g.T, size=256, replace=False))
    say(f"MXFP6 layer parity long, {len(tokens)} sampled tokens of {g.T}")
    layer_check(g, tokens=tokens)


@pytest.mark.parametrize("T,E,k,nr,H,I", [
    (1, 16, 4, 10, 512, 512),
    (70, 12, 6, 3, 512, 512),     # padding picks
    (300, 8, 2, 5, 512, 512),     # many 16-column blocks per slot
    (9, 8, 2, 6, 1024, 1536),     # several super-chunks, I past one scale group
    (3, 6, 2, 4, 15872, 512),     # largest H whose scale rows stage in LDS
    (40, 16, 12, 14, 512, 512),   # k = 12
    (511, 16, 4, 10, 512, 512),   # 2044 assignments: largest batch on the small-batch kernels
    (512, 16, 4, 10, 512, 512),   # 2048: smallest batch on the pipelined kernels
    (515, 12, 4, 7, 512, 512),    # pipelined: several 128-row tiles, ragged last tile
    (600, 6, 6, 6, 1024, 512),    # every expert picked by every token: 600 rows per slot
    (520, 8, 4, 6, 1536, 1024),   # pipelined: three scale groups for gate/up, two for down
    (200, 40, 12, 30, 512, 512),  # pipelined with k = 12
    (130, 20, 16, 18, 2048, 512),  # pipelined, a 16-row h pair per 64-row N-tile, K = 2048
])
def test_mxfp6_edge_shapes(T, E, k, nr, H, I):
    say(f"MXFP6 layer edge T={T} E={E} k={k} routable={nr} H={H} I={I}")
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=I, n_routable=nr, seed=T + 5 * E,
                              bias_scale=0.5)
    layer_check(GpuLayer(lay, act_format=FP6))


@pytest.mark.parametrize("T", [40, 600])
def test_mxfp6_shared_expert(T):
    say(f"MXFP6 layer with a shared expert, T={T}")
    lay = fixtures.tiny_layer(T=T, H=512, E=16, k=4, I=512, n_routable=10, seed=77,
                              bias_scale=0.5)
    g = GpuLayer(lay)
    from resident_expert_routing_amd import runtime as R
    import torch
    g.buf = R.LayerBuffers(g.T, g.H, g.E, g.k, g.I, g.S, torch.device("cuda", 0), shared=True,
                           act_format=FP6)
    wg, wu, wd = fixtures.expert_weights(43, 999, g.H, g.I)
    layer_check(g, shared=fixtures.pack_expert(wg, wu, wd))


def test_mxfp6_closer_to_unquantised_than_mxfp4():
    """The variant's point: against the layer with unquantised (bf16)
    activations, the MXFP6 run's error is well below the MXFP4 run's."""
    lay = fixtures.make_layer("decode")
    outs = {}
    for fmt in (0, FP6):
        g = GpuLayer(lay, act_format=fmt)
        g.route()
        g.experts()
        outs[fmt] = g.out_f64()
    r = oracle_route(g)
    ref, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                                 g.slot_bytes_fn(), g.H, g.I, act="bf16")
    e4, e6 = moe.rel_l2(outs[0], ref), moe.rel_l2(outs[FP6], ref)
    say(f"  rel-L2 to the unquantised layer: MXFP4 {e4:.3e}, MXFP6 {e6:.3e}")
    assert e6 < 0.5 * e4, (e4, e6)


def test_mxfp6_noalloc_matches():
    """The no-allocation entry point with MXFP6 rows gives the same bits."""
    import torch
    from resident_expert_routing_amd import binding as B
    lay = fixtures.make_layer("decode")
    g = GpuLayer(lay, act_format=FP6)
    g.route()
    g.experts()
    want = g.buf.out.cpu().numpy().copy()
    g.buf.out.zero_()
    b = g.buf
    B.check(B.moe_experts_forward_noalloc(b.T, b.H, b.I, b.k, b.S, b.xq, g.arena.mem,
                                          g.arena.stride, b.slot_offsets, b.perm, b.sel_slot,
                                          b.sel_weight, b.out, act_format=FP6),
            "moe_experts_forward_noalloc")
    torch.cuda.synchronize()
    assert np.array_equal(b.out.cpu().numpy(), want)


@pytest.mark.parametrize("name", ["prefill", "decode"])
def test_mxfp6_deferred_slot_same_output(name):
    """A deferred slot (its gate/up tiles after an event) gives the same bits."""
    import torch
    from resident_expert_routing_amd import runtime as R
    g = GpuLayer(fixtures.make_layer(name), act_format=FP6)
    say(f"MXFP6 deferred slot on {name}")
    g.route()
    g.experts()
    ref = g.out_f64().copy()
    counts = np.diff(g.routing()["slot_offsets"].astype(np.int64)[:g.S + 1])
    busiest = int(np.argmax(counts))
    small = int(np.flatnonzero((counts > 0) & (counts <= 128))[0])
    ev = torch.cuda.Event()
    for s in (busiest, small):
        ev.record()
        g.buf.out.zero_()
        R.experts(g.buf, g.arena.ptr(), g.arena.stride, defer_slot=s, defer_event=ev)
        assert np.array_equal(g.out_f64(), ref), (name, s, int(counts[s]))


def test_mxfp6_families_agree():
    """The same 255 tokens alone (small-batch kernels) and as the first rows of
    a 512-token batch (pipelined kernels) agree within the layer bar."""
    lay = fixtures.tiny_layer(T=512, H=512, E=16, k=4, I=512, n_routable=10, seed=93,
                              bias_scale=0.5)
    say("MXFP6 small-batch against pipelined kernels on the same tokens")
    full = GpuLayer(lay, act_format=FP6)
    full.route()
    full.experts()
    part = GpuLayer(lay, T=255, x_bits=lay.x_bits[:255], arena=full.arena, act_format=FP6)
    part.route()
    part.experts()
    a, b = part.out_f64(), full.out_f64()[:255]
    per = np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-300)
    say(f"  max per-token rel-L2 between families {per.max():.3e}")
    assert per.max() <= 2 * OUT_REL_L2
