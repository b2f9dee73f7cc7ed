"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: routing picks, slots, offsets, permutation and MXFP4 activation bytes
bit-exact; scores and renormalised weights within 1e-6; demand within 1e-5
relative per bin (exact zeros where nothing was picked); layer output within
relative L2 error 5e-3 of the float64 oracle.
"""
import numpy as np
import pytest

import fixtures
from oracle import moe, mxfp4
from gpu_helpers import GpuLayer, say, to_dev

pytestmark = pytest.mark.gpu

OUT_REL_L2 = 5e-3
DEMAND_REL = 1e-5
WEIGHT_ABS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import resident_expert_routing_amd  # noqa: F401  (loads libmoe_arena.so)
    from test_abi import hip_runtimes_mapped
    assert len(hip_runtimes_mapped()) == 1, hip_runtimes_mapped()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


_LAYERS = {}


def gpu_layer(name, T=None):
    key = (name, T)
    if key not in _LAYERS:
        say(f"workload {name} T={T}: generating inputs and uploading the arena")
        lay = fixtures.make_layer(name, T=T)
        _LAYERS[key] = GpuLayer(lay)
    return _LAYERS[key]


def oracle_route(g):
    r = moe.route(g.x_bits, g.lay.w_router, g.lay.bias, g.expert_slot_np, g.k)
    _, offsets, perm = moe.bucket(r["sel_slot"], g.S)
    r["slot_offsets"], r["perm"] = offsets, perm
    return r


def check_route(g, r):
    got = g.routing()
    for key in ("topk_expert", "sel_expert", "sel_slot", "slot_offsets", "perm"):
        assert np.array_equal(got[key], r[key]), key
    np.testing.assert_allclose(got["topk_score"], r["topk_score"], rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(got["sel_weight"], r["sel_weight"], rtol=0, atol=WEIGHT_ABS)
    H = g.H
    if g.T:
        codes, scales = mxfp4.encode(moe.bf16_to_f64(g.x_bits))
        assert np.array_equal(got["xq"][:, :H // 2], codes), "xq codes"
        assert np.array_equal(got["xq"][:, H // 2:H // 2 + H // 32], scales), "xq scales"
    return got


# --------------------------------------------------------------------------
# hardware probe: every E2M1 code at every scale whose result is a normal fp32,
# for both block-scaled instructions the expert kernels use
# --------------------------------------------------------------------------
# shape -> (output side n, lanes per K block): 0 = 16x16x128, 1 = 32x32x64
SHAPES = {0: 16, 1: 32}


def _probe(shape, a_codes, a_scale, b_codes, b_scale):
    """Codes [64 lanes][32] (values 0..15), scales [64] -> lane outputs [64][16]."""
    import torch
    import resident_expert_routing_amd as m
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    A = to_dev(pack(a_codes))
    Bq = to_dev(pack(b_codes))
    sa = to_dev(np.asarray(a_scale, dtype=np.uint8))
    sb = to_dev(np.asarray(b_scale, dtype=np.uint8))
    d = torch.zeros((64, 16), dtype=torch.float32, device=A.device)
    m.check(m.moe_test_mxfp4_probe(shape, A, sa, Bq, sb, d))
    torch.cuda.synchronize()
    return d.cpu().numpy()


def lane_matrix(shape, d):
    """Lane outputs -> D[n][n].  16x16x128: lane l, reg v = D[4*(l//16)+v][l%16];
    32x32x64: lane l, reg v = D[8*(v//4) + 4*(l//32) + v%4][l%32]."""
    n = SHAPES[shape]
    D = np.zeros((n, n), dtype=np.float32)
    for l in range(64):
        if shape == 0:
            for v in range(4):
                D[4 * (l // 16) + v, l % 16] = d[l, v]
        else:
            for v in range(16):
                D[8 * (v // 4) + 4 * (l // 32) + v % 4, l % 32] = d[l, v]
    return D


def kpos(shape):
    """A row i holds 1.0 at K position k_i (every row a different one)."""
    n = SHAPES[shape]
    nb = 64 // n   # K blocks per instruction
    return [32 * (i % nb) + (nb * (i // nb)) % 32 + 1 for i in range(n)]


def one_hot_rows(shape):
    n = SHAPES[shape]
    a = np.zeros((64, 32), dtype=np.uint8)
    for i, kk in enumerate(kpos(shape)):
        a[n * (kk // 32) + i, kk % 32] = 2      # lane n*block + row holds that block
    return a


def ramp_cols(shape):
    n = SHAPES[shape]
    b = np.zeros((64, 32), dtype=np.uint8)
    for l in range(64):
        j, g = l % n, l // n
        for m_ in range(32):
            b[l, m_] = (j + 32 * g + m_) % 16
    return b


@pytest.mark.parametrize("shape", [0, 1])
def test_probe_every_code_and_scale(shape):
    n = SHAPES[shape]
    say(f"probe shape {shape}: one-hot A against B codes (j+k)%16, B scales 2..250")
    a_codes, b_codes = one_hot_rows(shape), ramp_cols(shape)
    ks = kpos(shape)
    assert len(set(ks)) == n and max(ks) < 2048 // n
    for s in range(2, 251):
        D = lane_matrix(shape, _probe(shape, a_codes, [127] * 64, b_codes, [s] * 64))
        for i, kk in enumerate(ks):
            for j in range(n):
                want = mxfp4.VALUE[(j + kk) % 16] * 2.0 ** (s - 127)
                assert D[i, j] == np.float32(want), (s, i, j, D[i, j], want)
    say(f"probe shape {shape}: A-side decode (B one-hot)")
    for s in (2, 60, 127, 200, 250):
        D = lane_matrix(shape, _probe(shape, b_codes, [s] * 64, a_codes, [127] * 64))
        for j, kk in enumerate(ks):
            for i in range(n):
                want = mxfp4.VALUE[(i + kk) % 16] * 2.0 ** (s - 127)
                assert D[i, j] == np.float32(want)


@pytest.mark.parametrize("shape", [0, 1])
def test_probe_full_contraction(shape):
    n = SHAPES[shape]
    kdim = 2048 // n
    say(f"probe shape {shape}: random {n}x{n}x{kdim} contraction")
    rng = np.random.default_rng(shape)
    a = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
    b = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
    sa = rng.integers(120, 134, size=64)
    sb = rng.integers(120, 134, size=64)
    D = lane_matrix(shape, _probe(shape, a, sa, b, sb))
    # A[i][k], k = 32*g + m held by lane n*g+i; B[k][j] by lane n*g+j
    Am = np.zeros((n, kdim))
    Bm = np.zeros((kdim, n))
    for l in range(64):
        i, g = l % n, l // n
        Am[i, 32 * g:32 * g + 32] = mxfp4.VALUE[a[l]] * 2.0 ** (sa[l] - 127)
        Bm[32 * g:32 * g + 32, i] = mxfp4.VALUE[b[l]] * 2.0 ** (sb[l] - 127)
    want = Am @ Bm   # exact in float64 for these ranges
    bound = 8 * 2.0 ** -24 * (np.abs(Am) @ np.abs(Bm))   # a few fp32 roundings inside
    assert np.all(np.abs(D - want) <= bound)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "long"])
def test_route_parity(name):
    g = gpu_layer(name)
    say(f"moe_route parity on {name}: T={g.T} H={g.H} E={g.E} k={g.k} S={g.S}")
    g.route()
    check_route(g, oracle_route(g))


def test_route_worked_example_ties():
    """Exact ties (one-hot tokens) resolve to the lower expert id, on the GPU."""
    import torch
    from resident_expert_routing_amd import runtime as R
    say("moe_route on the hand-worked tie example")
    E, H, k = 6, 32, 3
    w = np.zeros((E, H), dtype=np.float32)
    w[:, 0] = [0.5, 2.0, 1.0, 2.0, -1.0, 1.5]
    w[:, 1] = [3.0, 0.0, 0.0, 1.0, 2.5, -2.0]
    x = np.zeros((2, H), dtype=np.float32)
    x[0, 0] = x[1, 1] = 1.0
    es = np.array([0, -1, 1, 2, -1, 3], dtype=np.int32)
    buf = R.LayerBuffers(2, H, E, k, 32, 4, torch.device("cuda", 0))
    R.route(buf, to_dev(fixtures.f32_to_bf16_bits(x).view(np.int16)), to_dev(w), None, to_dev(es))
    torch.cuda.synchronize()
    assert buf.topk_expert.cpu().numpy().tolist() == [[1, 3, 5], [0, 3, 4]]
    assert buf.sel_expert.cpu().numpy().tolist() == [[2, 3, 5], [0, 2, 3]]
    assert buf.sel_slot.cpu().numpy().tolist() == [[1, 2, 3], [0, 1, 2]]
    assert buf.slot_offsets.cpu().numpy().tolist() == [0, 1, 3, 5, 6]
    assert buf.perm.cpu().numpy().tolist() == [3, 0, 4, 1, 5, 2]


@pytest.mark.parametrize("T,E,k", [(40, 32, 4), (300, 32, 4), (9, 200, 8)])
def test_route_reuse_logits(T, E, k):
    """A second moe_route over a changed routable set with the router's products
    reused gives exactly what a fresh call over that set gives (fused path for
    T <= 64, multi-kernel path above)."""
    import torch
    from resident_expert_routing_amd import runtime as R
    say(f"moe_route reuse_logits T={T} E={E} k={k}")
    H = 256
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=32, n_routable=E // 2, seed=T + E,
                              bias_scale=0.5)
    S = E // 2
    es1 = lay.expert_slot.copy()
    dev = torch.device("cuda", 0)
    buf = R.LayerBuffers(T, H, E, k, 32, S, dev)
    x = to_dev(lay.x_bits.view(np.int16))
    w, b = to_dev(lay.w_router), to_dev(lay.bias)
    keys = ("topk_expert", "topk_score", "sel_expert", "sel_weight", "sel_slot",
            "slot_offsets", "perm", "xq")

    def outputs():
        torch.cuda.synchronize()
        return {key: getattr(buf, key).cpu().numpy().copy() for key in keys}

    # a hot read's table change: the most picked routable expert leaves, a
    # non-routable one takes its slot
    R.route(buf, x, w, b, to_dev(es1))
    picks = outputs()["sel_expert"]
    gone = int(np.bincount(picks[picks >= 0], minlength=E).argmax())
    came = int(np.flatnonzero(es1 < 0)[0])
    es2 = es1.copy()
    es2[came], es2[gone] = es1[gone], -1
    R.route(buf, x, w, b, to_dev(es2))
    fresh = outputs()
    R.route(buf, x, w, b, to_dev(es1))
    first = outputs()
    R.route(buf, x, w, b, to_dev(es2), reuse_logits=True)
    again = outputs()
    for key in keys:
        assert np.array_equal(again[key], fresh[key]), key
    assert not np.array_equal(first["sel_slot"], fresh["sel_slot"]), "the table change mattered"


@pytest.mark.parametrize("T,E,k,nr,S,H", [
    (1, 16, 4, 10, 10, 256),     # single token
    (13, 16, 4, 10, 10, 256),    # ragged token count
    (70, 40, 6, 3, 3, 96),       # fewer routable than k: padding; H not a multiple of 128
    (65, 16, 4, 16, 16, 256),    # all resident, T just above the split-router limit
    (5, 1024, 32, 700, 8192, 64),  # maximum E, k and S
    (9, 200, 8, 150, 8192, 128),   # fused selection + bucketing with the maximum S
    (16, 256, 8, 230, 230, 4096),  # four selection workgroups
    (17, 256, 8, 230, 230, 4096),  # a partly filled last selection workgroup
    (64, 256, 8, 230, 230, 4096),  # largest batch of the fused path
    (64, 256, 32, 250, 8192, 512),  # fused path: most assignments, maximum S
    (65, 256, 8, 230, 230, 4096),  # smallest batch of the multi-kernel path
    (8, 256, 32, 250, 8192, 512),  # one-launch decode path: most assignments, maximum S
    (3, 33, 6, 4, 40, 256),        # one-launch decode path: odd E, fewer routable than k
    (8, 256, 8, 230, 230, 4096),   # largest batch of the one-launch decode path
])
def test_route_edge_shapes(T, E, k, nr, S, H):
    say(f"moe_route edge T={T} E={E} k={k} routable={nr} S={S} H={H}")
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=32, n_routable=nr, seed=T * 7 + E,
                              bias_scale=0.5)
    es = lay.expert_slot.copy()
    if S > nr:   # spread the routable experts over a sparse slot range
        rng = np.random.default_rng(1)
        slots = rng.choice(S, size=nr, replace=False)
        es[es >= 0] = slots[es[es >= 0]]
    g = GpuLayer.__new__(GpuLayer)
    _init_route_only(g, lay, es, S)
    g.route()
    check_route(g, oracle_route(g))


@pytest.mark.parametrize("T,H,near", [(256, 512, False), (300, 1024, True), (2048, 4096, True)])
def test_route_certified_path_ties_and_near_ties(T, H, near):
    """Batches above 64 tokens with H a multiple of 512 route on bounded bf16
    logits and re-select, on float64 logits, every token whose k-th and
    (k+1)-th logits are within twice the bound.  Router rows repeated in
    groups of four make logits tie exactly in every token; with `near`, the
    repeats differ by j * 2^-20 in one weight, so the logits differ by far
    less than the bound.  Nearly every token then takes the second pass, and
    its picks -- exact ties to the lower expert id -- must be the oracle's.
    The weights are multiples of 2^-20 below 1, so every product and partial
    sum is exact in float64 and the oracle's ties do not depend on its
    summation order either."""
    E, k, nr = 64, 8, 40
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=128, n_routable=nr, seed=T + H,
                              bias_scale=0.0)
    w = (np.round(lay.w_router.astype(np.float64) * 4096) / 4096).astype(np.float32)
    for g in range(0, E, 4):
        w[g + 1:g + 4] = w[g]
        if near:
            for j in range(1, 4):
                w[g + j, j] += np.float32(j * 2.0 ** -20)
    lay.w_router = w
    lay.bias = np.zeros(E, dtype=np.float32)
    # activations below 2^-8 in magnitude are set to zero, so that a product's
    # lowest bit (>= 2^-35) and the largest partial sum (< 2^7) fit 53 bits
    xf = fixtures.bf16_bits_to_f32(lay.x_bits)
    lay.x_bits = np.where(np.abs(xf) < 2.0 ** -8, np.uint16(0), lay.x_bits).astype(np.uint16)
    say(f"certified routing: T={T} H={H}, router rows repeated in fours "
        f"({'near ties' if near else 'exact ties'})")
    g = GpuLayer(lay)
    g.route()
    check_route(g, oracle_route(g))


def _init_route_only(g, lay, es, S):
    import torch
    from resident_expert_routing_amd import runtime as R
    g.lay, g.x_bits, g.T = lay, lay.x_bits, lay.x_bits.shape[0]
    g.H, g.E, g.k, g.I, g.S = lay.cfg.H, lay.cfg.E, lay.cfg.k, lay.cfg.I, S
    g.expert_slot_np = es
    g.x = to_dev(lay.x_bits.view(np.int16))
    g.w_router, g.bias = to_dev(lay.w_router), to_dev(lay.bias)
    g.expert_slot = to_dev(es.astype(np.int32))
    g.buf = R.LayerBuffers(g.T, g.H, g.E, g.k, g.I, S, torch.device("cuda", 0))
    g.hist = torch.zeros(g.E, dtype=torch.float64, device=torch.device("cuda", 0))


@pytest.mark.parametrize("fill", ["random", "ones", "again"])
def test_route_decode_workspace_contents(fill):
    """The one-launch decode path keeps its completion counter in the
    workspace: whatever the workspace holds before the call (random bytes,
    all ones, the previous call's state), the picks, slots, bucketing and
    demand are the oracle's."""
    import torch
    lay = fixtures.tiny_layer(T=8, H=512, E=64, k=6, I=32, n_routable=40, seed=91,
                              bias_scale=0.5)
    g = GpuLayer.__new__(GpuLayer)
    _init_route_only(g, lay, lay.expert_slot.copy(), 40)
    ws = g.buf.ws_route
    if fill == "random":
        gen = torch.Generator(device="cpu").manual_seed(5)
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=gen).to(ws.device))
    elif fill == "ones":
        ws.fill_(255)
    else:
        g.route()
    from resident_expert_routing_amd import runtime as R
    say(f"decode routing with a workspace of {fill} contents")
    g.hist.zero_()
    R.route(g.buf, g.x, g.w_router, g.bias, g.expert_slot, hist_row=g.hist)
    torch.cuda.synchronize()
    r = oracle_route(g)
    check_route(g, r)
    want = moe.demand(r["topk_expert"], r["topk_score"], g.E)
    hist = g.hist.cpu().numpy()
    nz = want > 0
    assert (hist[~nz] == 0).all()
    assert np.all(np.abs(hist[nz] - want[nz]) <= DEMAND_REL * want[nz])


def test_route_empty_batch():
    import torch
    from resident_expert_routing_amd import runtime as R
    say("moe_route with T=0")
    buf = R.LayerBuffers(0, 256, 16, 4, 128, 10, torch.device("cuda", 0))
    buf.slot_offsets.fill_(77)
    x = torch.empty((0, 256), dtype=torch.int16, device="cuda")
    R.route(buf, x, torch.zeros((16, 256), device="cuda"), None,
            torch.zeros(16, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert (buf.slot_offsets.cpu().numpy() == 0).all()


# --------------------------------------------------------------------------
# demand
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_demand_parity(name):
    import torch
    g = gpu_layer(name)
    say(f"moe_demand_accumulate parity on {name}")
    g.route()
    g.hist.zero_()
    g.demand()
    g.demand()   # accumulates: hist = 2 * delta
    torch.cuda.synchronize()
    r = oracle_route(g)
    want = moe.demand(r["topk_expert"], r["topk_score"], g.E)
    delta = g.buf.delta.cpu().numpy().astype(np.float64)
    hist = g.hist.cpu().numpy()
    nz = want > 0
    assert (delta[~nz] == 0).all() and (hist[~nz] == 0).all()
    assert np.all(np.abs(delta[nz] - want[nz]) <= DEMAND_REL * want[nz])
    assert np.all(np.abs(hist[nz] - 2 * want[nz]) <= DEMAND_REL * 2 * want[nz])
    # demand totals equal the sum of the recorded (float32) scores, up to float64
    # summation order; and the oracle's float64 scores up to float32 rounding (2^-24 each)
    rec = g.buf.topk_score.cpu().numpy().astype(np.float64).sum()
    assert abs(hist.sum() - 2 * rec) <= 1e-12 * hist.sum()
    assert abs(hist.sum() - 2 * r["topk_score"].sum()) <= 2.0 ** -23 * hist.sum()


# --------------------------------------------------------------------------
# whole layer
# --------------------------------------------------------------------------
def _layer_parity(g, tokens=None):
    g.route()
    g.experts()
    out = g.out_f64()
    r = oracle_route(g)
    check_route(g, r)
    o, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                               g.slot_bytes_fn(), g.H, g.I, tokens=tokens)
    got = out if tokens is None else out[tokens]
    err = moe.rel_l2(got, o)
    say(f"  rel-L2 {err:.3e} over {got.shape[0]} tokens")
    assert err <= OUT_REL_L2, err
    return err


def test_layer_parity_tiny():
    say("layer parity tiny (all 64 tokens)")
    _layer_parity(gpu_layer("tiny"))


def test_layer_parity_decode():
    say("layer parity decode (all 8 tokens, ring slots routable)")
    _layer_parity(gpu_layer("decode"))


# Per-token bound.  A token's output carries two bf16 roundings (its y rows on
# the pipelined path, then out), each at most 2^-9 relative per element, so a
# token's own rel-L2 sits near the pooled figure.  One rare event moves a
# single token further: an element of h whose float32 value and the oracle's
# float64 value fall on two sides of an E2M1 rounding edge takes the
# neighbouring code.  That changes one of the token's y rows by one code step
# (at most 2X of a block whose amax is at least 4X) times one column of the
# down weights: relative to the row, at most about 2 / sqrt(I/32 blocks x 32)
# ~ 4.4e-2 at I = 2048, weighted by the pick's share of the output.  So every
# token must lie within 5e-2, and tokens above the pooled bar must be rare.
TOKEN_REL_L2_MAX = 5e-2
TOKEN_OVER_BAR_FRAC = 5e-3


def _layer_parity_all_tokens(g):
    """Every token: pooled rel-L2 <= 5e-3, each token <= 5e-2, and at most
    0.5 % of tokens above 5e-3."""
    g.route()
    g.experts()
    out = g.out_f64()
    r = oracle_route(g)
    check_route(g, r)
    o, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                               g.slot_bytes_fn(), g.H, g.I)
    err = moe.rel_l2(out, o)
    per = np.linalg.norm(out - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-300)
    over = int((per > OUT_REL_L2).sum())
    say(f"  pooled rel-L2 {err:.3e} over {g.T} tokens; per token: median {np.median(per):.3e}, "
        f"p99 {np.quantile(per, 0.99):.3e}, max {per.max():.3e} (token {int(per.argmax())}), "
        f"{over} above {OUT_REL_L2}")
    assert err <= OUT_REL_L2, err
    assert per.max() <= TOKEN_REL_L2_MAX, (per.max(), int(per.argmax()))
    assert over <= TOKEN_OVER_BAR_FRAC * g.T, over
    return err


@pytest.mark.timeout(600)
def test_layer_parity_prefill_all_tokens():
    g = gpu_layer("prefill")
    say(f"layer parity prefill, all {g.T} tokens (every M-tile and N-tile of every slot)")
    _layer_parity_all_tokens(g)


@pytest.mark.timeout(900)
def test_layer_parity_long_all_tokens():
    g = gpu_layer("long")
    say(f"layer parity long, all {g.T} tokens (every M-tile and N-tile of every slot)")
    _layer_parity_all_tokens(g)


@pytest.mark.parametrize("T", [8, 2048])
def test_layer_distinct_contents(T):
    """Every routable expert holds its own weights (no shared contents), at the
    decode and prefill workloads' expert and slot counts (256 experts, 166
    resident + 64 ring slots, top-8) with a smaller hidden size: a kernel that
    reads the wrong slot fails here with certainty."""
    say(f"layer with 230 distinct expert contents, T={T}")
    lay = fixtures.tiny_layer(T=T, H=512, E=256, k=8, I=512, n_routable=230, seed=71 + T,
                              bias_scale=0.5)
    assert lay.cfg.n_contents == 256
    _layer_parity_all_tokens(GpuLayer(lay))


@pytest.mark.parametrize("T,E,k,nr,H,I", [
    (1, 16, 4, 10, 256, 128),
    (13, 16, 4, 10, 256, 128),
    (70, 12, 6, 3, 96, 64),      # padding picks; partial 512-wide super-chunks
    (40, 8, 2, 8, 544, 160),     # H, I not multiples of 128
    (300, 8, 2, 5, 256, 128),    # small-batch kernels, many 16-column tiles per slot
    (129, 4, 1, 2, 544, 96),     # partial super-chunks in both GEMMs
    (511, 16, 4, 10, 512, 512),  # 2044 assignments: largest batch on the small-batch kernels
    (512, 16, 4, 10, 512, 512),  # 2048 assignments: smallest batch on the pipelined kernels
    (515, 12, 4, 7, 512, 512),   # pipelined: several 128-row tiles, ragged last tile
    (600, 6, 6, 6, 1024, 512),   # every expert picked by every token: 600 rows per slot
    (9, 8, 2, 6, 512, 96),       # small batch, gate/up scales staged in LDS, ragged I (idle wave)
    (17, 8, 2, 6, 800, 512),     # small batch, down scales staged, last 256-row block of 32 rows
    (3, 6, 2, 4, 8192, 64),      # H past the LDS scale-staging limit: scales read per super-chunk
    (520, 8, 4, 6, 768, 256),    # 2080 assignments, H not a multiple of 512: small-batch kernels
    (520, 8, 4, 6, 1536, 1024),  # pipelined: three scale groups for gate/up, two for down
    (40, 16, 12, 14, 256, 128),  # k = 12: the combine adds a batch of 8 picks, then one of 4
    (20, 40, 32, 36, 256, 128),  # k = 32 (the maximum): four batches of 8 picks
    (200, 40, 12, 30, 512, 512),  # pipelined (2400 assignments) with k = 12, bf16 y rows
])
def test_layer_edge_shapes(T, E, k, nr, H, I):
    say(f"layer edge T={T} E={E} k={k} routable={nr} H={H} I={I}")
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=I, n_routable=nr, seed=T + 3 * E,
                              bias_scale=0.5)
    _layer_parity(GpuLayer(lay))


@pytest.mark.parametrize("shared", [False, True])
def test_layer_sparse_slots_by_position(shared):
    """More than 1024 slots: a work item of the small-batch kernels is a
    position of the bucketed order, busy when it is its slot's first position;
    with a shared expert, its item follows all T*k positions."""
    say(f"layer with 12 routable experts spread over 2000 slots, shared expert: {shared}")
    T, H, E, k, I, S = 24, 256, 16, 4, 128, 2000
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=I, n_routable=12, seed=31, bias_scale=0.5)
    rng = np.random.default_rng(2)
    spread = rng.choice(S, size=12, replace=False)
    es = lay.expert_slot.copy()
    es[es >= 0] = spread[es[es >= 0]]
    slot_expert = np.full(S, -1)
    slot_expert[es[es >= 0]] = np.flatnonzero(es >= 0)
    lay.slot_expert = slot_expert.astype(np.int32)
    g = GpuLayer.__new__(GpuLayer)
    _init_route_only(g, lay, es, S)
    from resident_expert_routing_amd import runtime as R
    import torch
    g.arena = R.Arena(S, H, I, torch.device("cuda", 0))
    g.arena.mem.zero_()
    g.arena.upload(lambda s: lay.expert_bytes(slot_expert[s]), slots=spread)
    g.slot_bytes_fn = lambda: (lambda s: lay.expert_bytes(slot_expert[s]))
    if not shared:
        _layer_parity(g)
        return
    wg, wu, wd = fixtures.expert_weights(41, 999, H, I)
    sb = fixtures.pack_expert(wg, wu, wd)
    g.buf = R.LayerBuffers(T, H, E, k, I, S, torch.device("cuda", 0), shared=True)
    g.route()
    R.experts(g.buf, g.arena.ptr(), g.arena.stride, shared_expert=to_dev(sb))
    out = g.out_f64()
    r = oracle_route(g)
    check_route(g, r)
    o, _ = moe.experts_forward(g.x_bits, r["sel_expert"], r["sel_weight"], r["sel_slot"],
                               g.slot_bytes_fn(), H, I, shared_bytes=sb)
    err = moe.rel_l2(out, o)
    per = np.linalg.norm(out - o, axis=1) / np.maximum(np.linalg.norm(o, axis=1), 1e-300)
    say(f"  rel-L2 {err:.3e}, max per token {per.max():.3e}")
    assert err <= OUT_REL_L2 and per.max() <= TOKEN_REL_L2_MAX


def test_layer_sparse_slots_tiled():
    """Pipelined path with used slots spread over 3000 slot ids."""
    say("pipelined layer with 12 routable experts spread over 3000 slots")
    T, H, E, k, I, S = 600, 512, 16, 4, 512, 3000
    lay = fixtures.tiny_layer(T=T, H=H, E=E, k=k, I=I, n_routable=12, seed=33, bias_scale=0.5)
    rng = np.random.default_rng(3)
    spread = rng.choice(S, size=12, replace=False)
    es = lay.expert_slot.copy()
    es[es >= 0] = spread[es[es >= 0]]
    slot_expert = np.full(S, -1)
    slot_expert[es[es >= 0]] = np.flatnonzero(es >= 0)
    lay.slot_expert = slot_expert.astype(np.int32)
    g = GpuLayer.__new__(GpuLayer)
    _init_route_only(g, lay, es, S)
    from resident_expert_routing_amd import runtime as R
    import torch
    g.arena = R.Arena(S, H, I, torch.device("cuda", 0))
    g.arena.mem.zero_()
    g.arena.upload(lambda s: lay.expert_bytes(slot_expert[s]), slots=spread)
    g.slot_bytes_fn = lambda: (lambda s: lay.expert_bytes(slot_expert[s]))
    _layer_parity(g)


def test_layer_nothing_routable():
    import torch
    say("layer with no routable expert (S=0): output is zero")
    lay = fixtures.tiny_layer(T=5, H=256, E=16, k=4, I=128, n_routable=0, seed=9)
    g = GpuLayer(lay)
    g.route()
    g.experts()
    assert (g.out_f64() == 0).all()
    got = g.routing()
    assert (got["sel_expert"] == -1).all() and (got["slot_offsets"] == 0).all()


# --------------------------------------------------------------------------
# metamorphic properties (no oracle needed)
# --------------------------------------------------------------------------
def test_determinism_and_batch_invariance():
    import torch
    g = gpu_layer("decode")
    say("determinism: decode layer twice")
    g.route()
    g.experts()
    a = g.out_f64().copy()
    g.route()
    g.experts()
    assert np.array_equal(a, g.out_f64())
    say("batch invariance: each decode token alone")
    for t in (0, 3, 7):
        one = GpuLayer(g.lay, x_bits=g.x_bits[t:t + 1], arena=g.arena)
        one.route()
        one.experts()
        assert np.array_equal(one.out_f64()[0], a[t]), t


def test_batch_invariance_pipelined_path():
    """A token's output is bit-identical whether it runs in the 2048-token
    batch or in a 256-token batch (both on the matrix-core router and the
    pipelined kernels); alone (the small-batch kernels) it agrees to the
    layer's tolerance."""
    g = gpu_layer("prefill")
    say("batch invariance: 256 prefill tokens vs the same tokens in the 2048-token batch")
    g.route()
    g.experts()
    full = g.out_f64().copy()
    sub = GpuLayer(g.lay, x_bits=g.x_bits[100:356], arena=g.arena)
    sub.route()
    sub.experts()
    assert np.array_equal(sub.routing()["topk_score"], g.routing()["topk_score"][100:356])
    assert np.array_equal(sub.out_f64(), full[100:356])
    for t in (0, 777, 2047):
        one = GpuLayer(g.lay, x_bits=g.x_bits[t:t + 1], arena=g.arena)
        one.route()
        one.experts()
        # each path rounds its fp32 sums differently (and so may round an h
        # element to a neighbouring E2M1 code): the outputs agree to the
        # layer's tolerance, not bit for bit
        assert moe.rel_l2(one.out_f64()[0], full[t]) <= OUT_REL_L2, t


@pytest.mark.parametrize("name", ["prefill", "decode", "long"])
def test_deferred_slot_same_output(name):
    """moe_experts_forward with a deferred slot (its gate/up tiles run after
    an event, the other slots' before) gives the same output bit for bit, for
    the busiest slot, the least used one and an unused one (long: 256-row
    M-tiles)."""
    import torch
    from resident_expert_routing_amd import runtime as R
    g = gpu_layer(name)
    say(f"deferred slot on {name}: same output as one pass")
    g.route()
    g.experts()
    ref = g.out_f64().copy()
    off = g.routing()["slot_offsets"].astype(np.int64)
    counts = np.diff(off[:g.S + 1])
    busiest = int(np.argmax(counts))
    used = np.flatnonzero(counts > 0)
    small = int(used[np.argmin(counts[used])])
    unused = np.flatnonzero(counts == 0)
    slots = [busiest, small] + ([int(unused[0])] if unused.size else [])
    ev = torch.cuda.Event()
    for s in slots:
        ev.record()
        g.buf.out.zero_()
        R.experts(g.buf, g.arena.ptr(), g.arena.stride, defer_slot=s, defer_event=ev)
        assert np.array_equal(g.out_f64(), ref), (name, s, int(counts[s]))


def test_scale_bump_doubles_expert():
    """Adding 1 to every E8M0 scale byte of an expert's down matrix doubles that
    expert's y exactly; with identical experts everywhere the output doubles."""
    import torch
    say("metamorphic: down-scale bump doubles the output (identical experts)")
    lay = fixtures.tiny_layer(T=16, H=256, E=8, k=2, I=128, n_routable=8, seed=21, n_contents=1)
    g = GpuLayer(lay)
    g.route()
    g.experts()
    base = g.out_f64().copy()
    sec = fixtures.SlotLayout(256, 128).sections
    so, ss = sec["down_scales"]
    mem = g.arena.mem.view(g.S, -1)
    mem[:, so:so + ss] += 1
    g.experts()
    bumped = g.out_f64()
    # out is bf16(sum w*y); doubling every y doubles the fp32 sum exactly
    assert np.array_equal(bumped, 2 * base)


@pytest.mark.parametrize("name,T", [("tiny", None), ("decode", None), ("prefill", None),
                                    ("prefill", 1000), ("long", None)])
def test_route_with_demand_equals_separate_call(name, T):
    """moe_route with hist_row gives bit-for-bit the demand of moe_demand_accumulate
    (larger batches: chunk sums beside the bucket counts, final sums beside the
    placement; T=1000 ends on a part chunk of 40 tokens)."""
    import torch
    from resident_expert_routing_amd import runtime as R
    g = gpu_layer(name, T=T)
    say(f"moe_route with fused demand on {name} T={g.T}")
    g.route()
    g.hist.zero_()
    g.demand()
    torch.cuda.synchronize()
    want_hist = g.hist.cpu().numpy().copy()
    want_delta = g.buf.delta.cpu().numpy().copy()
    g.hist.zero_()
    g.buf.delta.fill_(-1.0)
    R.route(g.buf, g.x, g.w_router, g.bias, g.expert_slot, hist_row=g.hist)
    torch.cuda.synchronize()
    assert np.array_equal(g.hist.cpu().numpy(), want_hist)
    assert np.array_equal(g.buf.delta.cpu().numpy(), want_delta)
    check_route(g, oracle_route(g))


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_stage_events_bracket_gateup(name):
    """Stage events 1 and 2 come from the gate/up kernel's own dispatch: they lie
    inside the call's other events, and recording them changes no result."""
    import torch
    from resident_expert_routing_amd import runtime as R
    g = gpu_layer(name)
    say(f"moe_experts_forward with stage events on {name}")
    g.route()
    stream = torch.cuda.current_stream()
    g.experts(stream)
    base = g.out_f64()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for e in evs:
        e.record(stream)  # creates the HIP events
    torch.cuda.synchronize()
    R.experts(g.buf, g.arena.ptr(), g.arena.stride, stream, evs)
    torch.cuda.synchronize()
    assert np.array_equal(g.out_f64(), base)
    t01, t12 = evs[0].elapsed_time(evs[1]), evs[1].elapsed_time(evs[2])
    t23, t34 = evs[2].elapsed_time(evs[3]), evs[3].elapsed_time(evs[4])
    assert t12 > 0.0
    assert min(t01, t23, t34) >= 0.0
    assert evs[0].elapsed_time(evs[4]) >= t12


@pytest.mark.parametrize("act", [0, 1])
def test_fused_down_combine_bit_identical(act):
    """Batches of up to 32 tokens run down and combine as one kernel; 33
    tokens take the two-kernel path.  The first 32 tokens give the same bits
    either way (same instruction sequence per y element, same fused
    multiply-adds in pick order)."""
    say(f"fused down+combine (T=32) against the two-kernel path (T=33), act_format {act}")
    lay = fixtures.tiny_layer(T=33, H=1024, E=64, k=8, I=512, n_routable=40, seed=57,
                              bias_scale=0.5)
    full = GpuLayer(lay, act_format=act)
    full.route()
    full.experts()
    part = GpuLayer(lay, T=32, x_bits=lay.x_bits[:32], arena=full.arena, act_format=act)
    part.route()
    part.experts()
    a = part.buf.out.cpu().numpy()
    b = full.buf.out.cpu().numpy()[:32]
    assert np.array_equal(a, b)
    if act == 0:  # MXFP6 parity of the fused path: the decode cases of test_gpu_mxfp6
        _layer_parity(part)
