"""GPU parity of the shared expert fused into moe_experts_forward (colibri
cluster page, shared-expert item: every row, unweighted, added at one fixed
point -- here after the routed picks).  Both kernel families, ragged shared
tiles, and a layer with nothing routable; every token against the oracle, and
a shared expert of zero weights leaves the output's bits unchanged.

Bars: output relative L2 <= 5e-3 pooled, every token <= 5e-2, at most 0.5 % of
tokens above 5e-3 (the per-token bound of the layer parity tests).
"""
import numpy as np
import pytest

import fixtures
from gpu_helpers import GpuLayer, say, to_dev
from oracle import moe

pytestmark = pytest.mark.gpu

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


def shared_bytes(H, I, seed):
    wg, wu, wd = fixtures.expert_weights(seed, 999, H, I)
    return fixtures.pack_expert(wg, wu, wd)


def run(g, shared):
    """Route, then the experts with the shared expert (or without: None);
    returns the bf16 output bits."""
    import torch
    from resident_expert_routing_amd import runtime as R
    buf = R.LayerBuffers(g.T, g.H, g.E, g.k, g.I, g.S, g.x.device, shared=shared is not None)
    g.buf = buf
    g.route()
    R.experts(buf, g.arena.ptr(), g.arena.stride,
              shared_expert=to_dev(shared) if shared is not None else None)
    torch.cuda.synchronize()
    return buf.out.cpu().numpy().copy()


def check(g, sb):
    bits = run(g, sb)
    got = (bits.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    r = moe.route(g.x_bits, g.lay.w_router, g.lay.bias, g.expert_slot_np, g.k)
    o, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                               g.slot_bytes_fn(), g.H, g.I, shared_bytes=sb)
    err = moe.rel_l2(got, o)
    per = np.linalg.norm(got - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-300)
    over = int((per > OUT_REL_L2).sum())
    say(f"  with the shared expert: pooled rel-L2 {err:.3e} over {g.T} tokens, max per token "
        f"{per.max():.3e}, {over} above {OUT_REL_L2}")
    assert err <= OUT_REL_L2
    assert per.max() <= TOKEN_REL_L2_MAX
    assert over <= TOKEN_OVER_BAR_FRAC * g.T


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_shared_expert_workloads_small(name):
    lay = fixtures.make_layer(name)
    say(f"shared expert, {name} workload")
    check(GpuLayer(lay), shared_bytes(lay.cfg.H, lay.cfg.I, 31))


@pytest.mark.timeout(600)
def test_shared_expert_prefill_all_tokens():
    lay = fixtures.make_layer("prefill")
    say("shared expert, prefill workload (pipelined kernels, 16 shared M-tiles)")
    check(GpuLayer(lay), shared_bytes(lay.cfg.H, lay.cfg.I, 32))


@pytest.mark.parametrize("T,E,k,nr,H,I", [
    (13, 16, 4, 10, 256, 128),   # small batch
    (515, 12, 4, 7, 512, 512),   # pipelined, ragged last shared tile (515 = 4 x 128 + 3)
    (9, 8, 2, 0, 256, 128),      # nothing routable: the shared expert alone
    (600, 6, 6, 0, 512, 512),    # nothing routable at a pipelined batch size
    (3, 6, 2, 4, 8192, 64),      # scales read per super-chunk (H past the staging limit)
])
def test_shared_expert_edge_shapes(T, E, k, nr, H, I):
    say(f"shared expert edge T={T} E={E} k={k} routable={nr} H={H} I={I}")
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=I, n_routable=nr, seed=T + 5 * E,
                              bias_scale=0.5)
    check(GpuLayer(lay), shared_bytes(H, I, T))


@pytest.mark.parametrize("T", [8, 600])
def test_zero_shared_expert_changes_no_bit(T):
    lay = fixtures.tiny_layer(T=T, H=512, E=12, k=4, I=512, n_routable=9, seed=77 + T,
                              bias_scale=0.5)
    g = GpuLayer(lay)
    plain = run(g, None)
    wg, wu, wd = fixtures.expert_weights(1, 0, 512, 512)
    zero = fixtures.pack_expert(0 * wg, 0 * wu, 0 * wd)
    assert np.array_equal(run(g, zero), plain)
    say(f"  T={T}: a zero shared expert leaves every output bit as it was")
