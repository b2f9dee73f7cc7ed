"""moe_experts_forward_noalloc (the library's own scratch, no workspace
argument) against moe_experts_forward on the same inputs, through the C ABI:
two calls in a row on one GPU, the second with a smaller batch, each output
identical bit for bit to the workspace entry point's (same kernels) and within
the layer bar (relative L2 5e-3) of the float64 oracle."""
import numpy as np
import pytest

import fixtures
from oracle import moe
from gpu_helpers import GpuLayer, say

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


def _both(g):
    """(out of moe_experts_forward, out of moe_experts_forward_noalloc) as bf16 bits."""
    import torch
    from resident_expert_routing_amd import binding as B
    g.route()
    b = g.buf
    B.check(B.moe_experts_forward(g.T, g.H, g.I, g.k, g.S, b.xq, g.arena.mem, g.arena.stride,
                                  b.slot_offsets, b.perm, b.sel_slot, b.sel_weight, b.out,
                                  b.ws_experts, b.ws_experts_bytes), "moe_experts_forward")
    torch.cuda.synchronize()
    ref = b.out.cpu().numpy().copy()
    b.out.fill_(0x7F7F)   # a value no result has: every element must be rewritten
    B.check(B.moe_experts_forward_noalloc(g.T, g.H, g.I, g.k, g.S, b.xq, g.arena.mem,
                                          g.arena.stride, b.slot_offsets, b.perm, b.sel_slot,
                                          b.sel_weight, b.out), "moe_experts_forward_noalloc")
    torch.cuda.synchronize()
    return ref, b.out.cpu().numpy().copy()


def _oracle_err(g, bits):
    r = moe.route(g.x_bits, g.lay.w_router, g.lay.bias, g.expert_slot_np, g.k)
    o, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                               g.slot_bytes_fn(), g.H, g.I)
    got = (bits.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return moe.rel_l2(got, o)


def test_noalloc_matches_workspace_entry_point_twice():
    big = fixtures.make_layer("decode")                 # 8 tokens, 230 slots
    say("no-alloc experts: decode batch (8 tokens), then 3 tokens of another batch")
    g1 = GpuLayer(big)
    ref, got = _both(g1)
    assert np.array_equal(ref, got), "first call differs from moe_experts_forward"
    err = _oracle_err(g1, got)
    say(f"  first call (T=8): identical to the workspace call; oracle rel-L2 {err:.3e}")
    assert err <= OUT_REL_L2

    small = fixtures.make_layer("decode", T=3, x_stream=5)
    g2 = GpuLayer(small, arena=g1.arena)               # same arena, smaller, different batch
    ref2, got2 = _both(g2)
    assert np.array_equal(ref2, got2), "second (smaller) call differs"
    err2 = _oracle_err(g2, got2)
    say(f"  second call (T=3): identical to the workspace call; oracle rel-L2 {err2:.3e}")
    assert err2 <= OUT_REL_L2


def test_noalloc_refuses_batches_past_its_scratch():
    import torch
    from resident_expert_routing_amd import binding as B
    T, H, k, I, S = 2048, 4096, 8, 2048, 166
    need = B.moe_workspace_bytes(B.MOE_OP_EXPERTS, T, H, 0, k, I, S)
    assert need > B.MOE_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(256, dtype=torch.uint8, device="cuda")
    st = B.moe_experts_forward_noalloc(T, H, I, k, S, dummy, dummy, B.moe_slot_bytes(H, I),
                                       dummy, dummy, dummy, dummy, dummy)
    assert st == B.MOE_ESCRATCH, B.status_string(st)
