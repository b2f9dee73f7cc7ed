"""Pins for the oracle's expert FFN, combine and whole-layer assembly (CPU only).

Brute force with Python scalar loops and math.fsum on tiny shapes, textbook
SwiGLU special cases, and the identical-experts invariant (when every routable
slot holds the same expert, the layer output is that expert's FFN of the
token, whatever the routing, because the renormalised weights sum to one).
"""
import math

import numpy as np

import fixtures
from oracle import moe, mxfp4


def _weights(H, I, seed):
    return fixtures.expert_weights(seed, 0, H, I)


def _quantise_scalar(vals):
    """Encode/decode one row via the oracle encoder (pinned in test_oracle_mxfp4)."""
    return list(mxfp4.quantise(np.array([vals], dtype=np.float64))[0])


def brute_ffn(xhat_row, wg, wu, wd):
    I, H = wg.shape
    g = [math.fsum(xhat_row[h] * wg[i, h] for h in range(H)) for i in range(I)]
    u = [math.fsum(xhat_row[h] * wu[i, h] for h in range(H)) for i in range(I)]
    h = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    hq = _quantise_scalar(h)
    return [math.fsum(hq[i] * wd[n, i] for i in range(I)) for n in range(wd.shape[0])]


def check_ffn_bruteforce():
    H, I = 64, 32
    for seed in range(3):
        buf = fixtures.pack_expert(*_weights(H, I, 50 + seed))
        W = moe.decode_expert(buf, H, I)
        x = fixtures.draw_tokens(seed, 3, H)
        xhat = moe.quantise_rows(moe.bf16_to_f64(x))
        y = moe.expert_ffn(xhat, W)
        for t in range(3):
            ref = brute_ffn(list(xhat[t]), *W)
            assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-15), seed


def test_ffn_bruteforce():
    check_ffn_bruteforce()


def test_silu_zero_and_zero_gate():
    assert moe.silu(np.array([0.0]))[0] == 0.0
    H, I = 64, 32
    wg, wu, wd = _weights(H, I, 60)
    W = moe.decode_expert(fixtures.pack_expert(np.zeros_like(wg), wu, wd), H, I)
    xhat = moe.quantise_rows(moe.bf16_to_f64(fixtures.draw_tokens(1, 4, H)))
    assert (moe.expert_ffn(xhat, W) == 0).all()
    W = moe.decode_expert(fixtures.pack_expert(wg, np.zeros_like(wu), wd), H, I)
    assert (moe.expert_ffn(xhat, W) == 0).all()


def test_k1_single_expert_is_textbook_swiglu():
    """k = 1 and one routable expert: the layer is that expert's SwiGLU MLP."""
    H, I, E = 64, 32, 5
    lay = fixtures.tiny_layer(T=6, H=H, E=E, k=1, I=I, n_routable=1, seed=12)
    buf = fixtures.pack_expert(*_weights(H, I, 70))
    r = moe.layer(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, 1, lambda s: buf, H, I,
                  act="bf16")
    wg, wu, wd = moe.decode_expert(buf, H, I)
    x = moe.bf16_to_f64(lay.x_bits)
    g = x @ wg.T
    textbook = (g * (1 / (1 + np.exp(-g))) * (x @ wu.T)) @ wd.T
    assert np.allclose(r["out"], textbook, rtol=1e-13, atol=1e-16)
    assert (r["sel_weight"][:, 0] == 1.0).all()


def check_identical_experts():
    H, I, E, k = 64, 32, 12, 4
    buf = fixtures.pack_expert(*_weights(H, I, 80))
    W = moe.decode_expert(buf, H, I)
    for seed, nr in ((1, 12), (2, 7), (3, 4)):
        lay = fixtures.tiny_layer(T=10, H=H, E=E, k=k, I=I, n_routable=nr, seed=seed, bias_scale=1.0)
        r = moe.layer(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, k, lambda s: buf, H, I)
        xhat = moe.quantise_rows(moe.bf16_to_f64(lay.x_bits))
        assert np.allclose(r["out"], moe.expert_ffn(xhat, W), rtol=1e-12, atol=1e-15)


def test_identical_experts_invariant():
    check_identical_experts()


def test_combine_order_and_padding():
    y = np.arange(2 * 3 * 4, dtype=np.float64).reshape(2, 3, 4)
    w = np.array([[0.5, 0.25, 0.25], [1.0, 0.0, 0.0]])
    se = np.array([[1, 2, 3], [4, -1, -1]])
    y[1, 1:] = np.nan    # padded picks are never read
    out = moe.combine(y, w, se)
    assert np.array_equal(out[0], 0.5 * y[0, 0] + 0.25 * y[0, 1] + 0.25 * y[0, 2])
    assert np.array_equal(out[1], y[1, 0])


def test_decode_expert_sections():
    H, I = 64, 32
    wg, wu, wd = _weights(H, I, 90)
    buf = fixtures.pack_expert(wg, wu, wd)
    g, u, d = moe.decode_expert(buf, H, I)
    assert g.shape == (I, H) and u.shape == (I, H) and d.shape == (H, I)
    # each decoded matrix is its float32 source quantised row-wise
    for got, src in ((g, wg), (u, wu), (d, wd)):
        assert np.array_equal(got, mxfp4.quantise(src.astype(np.float64)))
        assert np.abs(got - src).max() <= np.abs(src).max() / 2   # coarse but tight enough


def test_shared_expert_closed_forms():
    """Shared expert (colibri cluster page, shared-expert item: every row,
    unweighted, added at one fixed point):
    - every routed expert and the shared one identical -> out = 2 FFN(x^)
      for any routing and mask (the routed weights sum to 1);
    - a shared expert whose weights are all zero adds exactly nothing;
    - no routable expert at all -> out = the shared expert's FFN alone."""
    H, I, E, k = 64, 32, 12, 4
    buf = fixtures.pack_expert(*_weights(H, I, 81))
    W = moe.decode_expert(buf, H, I)
    zero = fixtures.pack_expert(*[np.zeros_like(w) for w in _weights(H, I, 1)])
    for seed, nr in ((4, 12), (5, 6)):
        lay = fixtures.tiny_layer(T=9, H=H, E=E, k=k, I=I, n_routable=nr, seed=seed,
                                  bias_scale=1.0)
        xhat = moe.quantise_rows(moe.bf16_to_f64(lay.x_bits))
        r = moe.layer(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, k, lambda s: buf, H, I,
                      shared_bytes=buf)
        assert np.allclose(r["out"], 2 * moe.expert_ffn(xhat, W), rtol=1e-12, atol=1e-15)
        other = fixtures.pack_expert(*_weights(H, I, 82 + seed))
        plain = moe.layer(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, k,
                          lambda s: other, H, I)
        with0 = moe.layer(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, k,
                          lambda s: other, H, I, shared_bytes=zero)
        assert np.array_equal(plain["out"], with0["out"])
    lay = fixtures.tiny_layer(T=5, H=H, E=E, k=k, I=I, n_routable=0, seed=6)
    r = moe.layer(lay.x_bits, lay.w_router, lay.bias, lay.expert_slot, k, lambda s: buf, H, I,
                  shared_bytes=buf)
    xhat = moe.quantise_rows(moe.bf16_to_f64(lay.x_bits))
    assert np.allclose(r["out"], moe.expert_ffn(xhat, W), rtol=1e-12, atol=1e-15)


def test_slot_code_tiles_hand_worked():
    """Code bytes of a slot section in tiles of 16 rows x 64 bytes, worked by
    hand for 32 rows of 80 code bytes (K = 160: one full tile and one 16-byte
    tile per row block):
      row 0, byte 0  -> 0;  row 1, byte 0 -> 64 (second row of the first tile);
      row 0, byte 64 -> 1024 (first row of the block's 16-byte tile);
      row 17, byte 70 -> 1280 (block 1) + 1024 + 1*16 + 6 = 2326;
      row 31, byte 79 -> 1280 + 1024 + 15*16 + 15 = 2559 (the last byte)."""
    pos = moe.code_position
    want = {(0, 0): 0, (1, 0): 64, (0, 64): 1024, (17, 70): 2326, (31, 79): 2559,
            (16, 0): 1280, (15, 63): 15 * 64 + 63}
    for (n, j), p in want.items():
        assert int(pos(np.array(n), np.array(j), 80)) == p, (n, j)
    # every byte lands once
    allp = pos(np.arange(32)[:, None], np.arange(80)[None, :], 80)
    assert sorted(allp.reshape(-1).tolist()) == list(range(32 * 80))
    # the packer puts byte (n, j) of its row-major codes where the formula says
    codes = (np.arange(32)[:, None] * 7 + np.arange(80)[None, :] * 3).astype(np.uint8)
    tiled = fixtures.tile_codes(codes)
    assert np.array_equal(tiled[allp], codes)
    # whole tiles only: a 64-byte tile of 16 rows is 1 KB, rows contiguous
    c2 = (np.arange(16)[:, None] * 5 + np.arange(128)[None, :]).astype(np.uint8)
    t2 = fixtures.tile_codes(c2)
    assert np.array_equal(t2[:1024].reshape(16, 64), c2[:, :64])
    assert np.array_equal(t2[1024:].reshape(16, 64), c2[:, 64:])
