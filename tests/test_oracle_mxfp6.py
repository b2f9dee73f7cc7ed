"""Pins for the oracle's MXFP6 (E2M3) decode and encode (CPU only).

Decode is checked exhaustively against the OCP MX v1.0 FP6 E2M3 value table
(literal magnitudes, not the bit-field formula the decoder uses); the bit
packing against a hand-worked block; encode against hand-derived ties and
scales, a round trip of every representable value at many scales, a literal
brute-force encoder on random blocks, and exact rational rounding over every
finite bf16 value of one scale window.
"""
from fractions import Fraction

import numpy as np
import pytest

import fixtures
from oracle import moe, mxfp6

# OCP MX v1.0, FP6 E2M3: magnitudes of codes 0..31 (codes 32..63 negate).
E2M3_TABLE = [0.0, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875,
              1.0, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875,
              2.0, 2.25, 2.5, 2.75, 3.0, 3.25, 3.5, 3.75,
              4.0, 4.5, 5.0, 5.5, 6.0, 6.5, 7.0, 7.5]


def test_decode_exhaustive():
    codes = np.concatenate([np.arange(32), np.arange(32, 64)]).astype(np.uint8)[None, :]
    packed = mxfp6.pack(codes)
    assert packed.shape == (1, 48)
    for s in range(255):
        vals = mxfp6.decode(packed, np.array([[s, s]], dtype=np.uint8))[0]
        for i, c in enumerate(codes[0]):
            mag = E2M3_TABLE[c & 31]
            want = (-mag if c & 32 else mag) * float(Fraction(2) ** (s - 127))
            assert vals[i] == want, (s, c)
    assert np.isnan(mxfp6.decode(packed[:, :24], np.array([[255]], dtype=np.uint8))).all()


def test_packing_hand_worked():
    """Element i at bits [6i, 6i+6) of the block's 24 bytes, little-endian.

    Codes 1, 2, 3, 4 then zeros: bits 0-5 = 000001, 6-11 = 000010, 12-17 =
    000011, 18-23 = 000100, so the 24-bit number is 0b000100_000011_000010_000001
    = 0x1030 81 -> bytes 0x81, 0x30, 0x10.  Code 63 as element 31 sets bits
    186-191: the top six bits of byte 23 (0xFC).
    """
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, :4] = [1, 2, 3, 4]
    codes[0, 31] = 63
    p = mxfp6.pack(codes)[0]
    assert p[:3].tolist() == [0x81, 0x30, 0x10]
    assert p[3:23].tolist() == [0] * 20 and p[23] == 0xFC
    assert np.array_equal(mxfp6.unpack(p[None, :]), codes)
    rng = np.random.default_rng(0)
    c = rng.integers(0, 64, size=(5, 96), dtype=np.uint8)
    assert np.array_equal(mxfp6.unpack(mxfp6.pack(c)), c)


def test_ties_to_even_mantissa_and_scale():
    """A block whose largest magnitude is 6 has X = 2^(floor(log2 6) - 2) = 1,
    so the other elements round on the E2M3 grid directly."""
    blk = np.zeros(32)
    blk[0] = 6.0
    cases = [
        (1.0625, 1.0),     # between 1.0 (m=0) and 1.125 (m=1): even -> 1.0
        (1.1875, 1.25),    # between 1.125 (m=1) and 1.25 (m=2)
        (0.0625, 0.0),     # subnormal tie 0 / 0.125
        (0.1875, 0.25),    # subnormal tie 0.125 / 0.25
        (0.9375, 1.0),     # 0.875 (e=0, m=7) / 1.0 (e=1, m=0)
        (3.875, 4.0),      # 3.75 (m=7) / 4.0 (next binade, m=0)
        (6.25, 6.0),       # 6.0 (m=4) / 6.5 (m=5)
        (-2.125, -2.0),    # 2.0 (m=0) / 2.25 (m=1), sign kept
        (1.2, 1.25),       # plain nearest
    ]
    for i, (v, _) in enumerate(cases):
        blk[1 + i] = v
    q = mxfp6.quantise(blk[None, :])[0]
    for i, (v, want) in enumerate(cases):
        assert q[1 + i] == want, (v, q[1 + i], want)
    # amax 8 -> X = 2: 8 -> 4 * 2; 7.5 -> 3.75 * 2 exactly; 0.2 -> 0.125 * 2 (0.1 -> 0.125)
    b2 = np.zeros((1, 32))
    b2[0, :3] = [8.0, 7.5, 0.2]
    p, s = mxfp6.encode(b2)
    assert s[0, 0] == 128
    assert mxfp6.decode(p, s)[0, :3].tolist() == [8.0, 7.5, 0.25]
    # saturation: amax 7.9 -> X = 1, 7.9 -> 7.5
    assert mxfp6.quantise(np.array([[7.9] + [0.0] * 31]))[0, 0] == 7.5
    # an all-zero block: scale byte 0, codes 0 (and negative zeros keep their sign bit)
    p, s = mxfp6.encode(np.zeros((1, 32)))
    assert s[0, 0] == 0 and (p == 0).all()


def test_round_trip_every_value_at_many_scales():
    rng = np.random.default_rng(1)
    for s in list(range(100, 155)) + [1, 254]:
        codes = rng.integers(0, 64, size=(4, 32), dtype=np.uint8)
        codes[:, 0] = 31                          # 7.5 sets the block's scale to s
        v = mxfp6.decode(mxfp6.pack(codes), np.full((4, 1), s, dtype=np.uint8))
        p, sc = mxfp6.encode(v)
        assert (sc == s).all()
        got = mxfp6.unpack(p)
        # +0 and -0 decode alike; every other code comes back
        same = (got == codes) | ((got & 31) == 0) & ((codes & 31) == 0)
        assert same.all()


def brute_encode_block(v):
    """Literal encoder: scale from amax, then every element tries all 64 codes."""
    amax = max(abs(x) for x in v)
    if amax == 0:
        return [0] * 32, 0
    e = max(-127, min(127, (np.frexp(amax)[1] - 1) - 2))   # floor(log2 amax) - 2, exactly
    X = 2.0 ** e
    out = []
    for x in v:
        best = None
        for c in range(64):
            val = mxfp6.e2m3_value(c) * X
            d = abs(val - x)
            key = (d, c & 1, 0 if (c >> 5) == (1 if np.signbit(x) else 0) else 1)
            if best is None or key < best[0]:
                best = (key, c)
        out.append(best[1])
    return out, e + 127


def test_encode_matches_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(40):
        v = rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20)
        if trial % 5 == 0:
            v[rng.integers(0, 32, size=4)] = 0.0
        p, s = mxfp6.encode(v[None, :])
        codes, sc = brute_encode_block(v)
        assert s[0, 0] == sc
        got = mxfp6.unpack(p)[0]
        for i in range(32):
            # a magnitude-0 result may carry either sign; all others must agree exactly
            if (codes[i] & 31) == 0:
                assert (got[i] & 31) == 0
            else:
                assert got[i] == codes[i], (trial, i, v[i], got[i], codes[i])


def test_bf16_window_exact_rounding():
    """Every finite bf16 value in [2^-4, 8) of a block whose scale is 1 (its
    largest element 7.5): rounded against exact rationals, ties to the even
    mantissa."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = (bits << 16).view(np.float32).astype(np.float64)
    sel = vals[np.isfinite(vals) & (np.abs(vals) >= 2.0 ** -4) & (np.abs(vals) < 8.0)]
    n = len(sel)
    rows = np.zeros((n, 32))
    rows[:, 0] = 7.5
    rows[:, 1] = sel
    q = mxfp6.quantise(rows)[:, 1]
    grid = [Fraction(m).limit_denominator(8) for m in E2M3_TABLE]
    for v, got in zip(sel, q):
        a = abs(Fraction(float(v)))
        d = [abs(a - g) for g in grid]
        best = min(d)
        cands = [i for i, x in enumerate(d) if x == best]
        i = min(cands, key=lambda i: (i & 1, i))
        want = float(grid[i]) * (-1 if v < 0 else 1)
        assert got == want, (v, got, want)


def test_quantise_rows_selects_format():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 64))
    assert np.array_equal(moe.quantise_rows(x, "mxfp6"), mxfp6.quantise(x))
    e6 = np.abs(moe.quantise_rows(x, "mxfp6") - x).max()
    e4 = np.abs(moe.quantise_rows(x, "mxfp4") - x).max()
    assert e6 < e4
    with pytest.raises(ValueError):
        moe.quantise_rows(x, "fp5")


def test_row_bytes():
    assert mxfp6.row_bytes(4096) == 3072 + 128
    assert fixtures is not None
