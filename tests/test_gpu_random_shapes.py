"""GPU parity over a seeded sweep of random layer shapes: batch sizes on both
sides of the kernel-family crossover (2048 assignments), expert counts, top-k,
routable counts (padding picks included) and hidden / intermediate sizes, in
both activation formats.  Each shape runs route + experts through the C ABI
and is compared with the oracle: routing outputs bit-exact, the activation
rows' bytes bit-exact, and the layer output within the layer bars (pooled
relative L2 <= 5e-3, every token <= 5e-2).

The shapes are drawn once from a fixed seed (numpy PCG64), so the sweep is
the same on every run; each case prints its shape before it runs.
"""
import numpy as np
import pytest

import fixtures
from gpu_helpers import GpuLayer, say
from oracle import moe, mxfp4, mxfp6

pytestmark = pytest.mark.gpu

OUT_REL_L2 = 5e-3
TOKEN_REL_L2_MAX = 5e-2


def _draw_shapes(n=24, seed=20261202):
    g = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        fmt = int(i % 2)                        # alternate MXFP4 / MXFP6
        if fmt == 1:                            # MXFP6: H, I multiples of 512
            H = int(g.choice([512, 1024, 1536, 2048]))
            I = int(g.choice([512, 1024]))
        else:
            H = int(32 * g.integers(2, 48))     # 64 .. 1504
            I = int(32 * g.integers(2, 40))     # 64 .. 1248
            if i % 4 == 0:                      # whole scale groups: the pipelined family can run
                H, I = 512 * int(g.integers(1, 4)), 512 * int(g.integers(1, 3))
        E = int(g.integers(4, 97))
        k = int(g.integers(1, min(E, 12) + 1))
        nr = int(g.integers(1, E + 1))          # routable experts (< k gives padding picks)
        # about half the cases past the crossover, the rest below it
        if i % 3 == 0:
            T = int(g.integers((2048 + k - 1) // k, (2048 + k - 1) // k + 300))
        else:
            T = int(g.integers(1, max(2, 2048 // k)))
        shapes.append((i, T, E, k, nr, H, I, fmt))
    return shapes


SHAPES = _draw_shapes()


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import resident_expert_routing_amd  # noqa: F401
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def test_sweep_covers_both_families_and_formats():
    fam = {(T * k >= 2048 and H % 512 == 0 and I % 512 == 0, fmt)
           for _, T, E, k, nr, H, I, fmt in SHAPES}
    assert fam == {(False, 0), (True, 0), (False, 1), (True, 1)}, fam
    assert any(nr < k for _, T, E, k, nr, H, I, fmt in SHAPES)


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: f"c{c[0]}")
def test_random_shape_parity(case):
    i, T, E, k, nr, H, I, fmt = case
    say(f"random shape {i}: T={T} E={E} k={k} routable={nr} H={H} I={I} "
        f"act={'mxfp6' if fmt else 'mxfp4'} (assignments {T * k})")
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=I, n_routable=nr, seed=1000 + i,
                              bias_scale=0.5)
    g = GpuLayer(lay, act_format=fmt)
    g.route()
    g.experts()
    out = g.out_f64()
    r = moe.route(g.x_bits, lay.w_router, lay.bias, g.expert_slot_np, k)
    _, offsets, perm = moe.bucket(r["sel_slot"], g.S)
    got = g.routing()
    for key, want in (("topk_expert", r["topk_expert"]), ("sel_expert", r["sel_expert"]),
                      ("sel_slot", r["sel_slot"]), ("slot_offsets", offsets), ("perm", perm)):
        assert np.array_equal(got[key], want), key
    np.testing.assert_allclose(got["sel_weight"], r["sel_weight"], rtol=0, atol=1e-6)
    xf = moe.bf16_to_f64(g.x_bits)
    if fmt:
        codes, scales = mxfp6.encode(xf)
        nc = 3 * H // 4
    else:
        codes, scales = mxfp4.encode(xf)
        nc = H // 2
    assert np.array_equal(got["xq"][:, :nc], codes), "xq codes"
    assert np.array_equal(got["xq"][:, nc:nc + H // 32], scales), "xq scales"
    o, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                               g.slot_bytes_fn(), H, I, act="mxfp6" if fmt else "mxfp4")
    err = moe.rel_l2(out, o)
    per = np.linalg.norm(out - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-300)
    say(f"  rel-L2 {err:.3e}, max per token {per.max():.3e}")
    assert err <= OUT_REL_L2, err
    assert per.max() <= TOKEN_REL_L2_MAX, (per.max(), int(per.argmax()))
