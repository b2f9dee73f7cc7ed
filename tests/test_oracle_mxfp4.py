"""Pins for the oracle's MXFP4 decode and encode (CPU only).

Decode is checked exhaustively against the OCP MX v1.0 E2M1 value table
(literal values, not the bit-field formula the decoder uses); encode against
hand-derived golden blocks, a round trip of every representable value at many
scales, and an exhaustive sweep of all finite bf16 values in one scale window
against exact rational rounding.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import fixtures
from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_blocks.txt")

# OCP MX v1.0, FP4 (E2M1) table: magnitudes for codes 0..7; codes 8..15 negate.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def check_decode_exhaustive():
    codes = np.arange(16, dtype=np.uint8)
    for s in range(255):
        # one block: codes 0..15 then 0..15 again
        row = np.concatenate([codes, codes])
        packed = (row[0::2] | (row[1::2] << 4)).astype(np.uint8)[None, :]
        vals = mxfp4.decode(packed, np.array([[s]], dtype=np.uint8))[0]
        for i, c in enumerate(row):
            mag = E2M1_TABLE[c & 7]
            want = (-mag if c & 8 else mag) * float(Fraction(2) ** (s - 127))
            assert vals[i] == want, (s, c, vals[i], want)
    nan = mxfp4.decode(np.array([[0x22] * 16], dtype=np.uint8), np.array([[255]], dtype=np.uint8))
    assert np.isnan(nan).all()


def test_decode_exhaustive():
    check_decode_exhaustive()


def test_negative_zero_decodes_to_zero():
    v = mxfp4.decode(np.array([[0x88] * 16], dtype=np.uint8), np.array([[127]], dtype=np.uint8))
    assert (v == 0).all()


def _parse(tok):
    tok = tok.strip()
    if "0x" in tok:
        return float.fromhex(tok)
    return float(tok)


def golden_blocks():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            name, vals, scale, codes = [p.strip() for p in line.split("|")]
            v = [_parse(t) for t in vals.split(",")]
            c = [int(t) for t in codes.split(",")]
            out.append((name, v, int(scale), c))
    return out


def check_encode_golden():
    for name, v, scale, codes in golden_blocks():
        blk = np.zeros((1, 32))
        blk[0, :len(v)] = v
        packed, sc = mxfp4.encode(blk)
        got = mxfp4.unpack_nibbles(packed)[0]
        assert int(sc[0, 0]) == scale, (name, sc[0, 0], scale)
        assert list(got[:len(codes)]) == codes, (name, list(got[:len(codes)]), codes)
        assert (got[len(codes):] == 0).all(), name


def test_encode_golden():
    check_encode_golden()


def test_packer_matches_golden_where_float32():
    for name, v, scale, codes in golden_blocks():
        if name == "clamp_high":
            continue  # 2**130 is not a float32
        blk = np.zeros((1, 32), dtype=np.float32)
        blk[0, :len(v)] = np.array(v, dtype=np.float64).astype(np.float32)
        if not np.array_equal(blk[0, :len(v)].astype(np.float64), np.array(v)):
            continue
        packed, sc = fixtures.pack_mxfp4_rows(blk)
        assert int(sc[0, 0]) == scale
        assert list(mxfp4.unpack_nibbles(packed)[0][:len(codes)]) == codes


def check_roundtrip():
    rng = np.random.default_rng(7)
    for e in range(-125, 126, 3):
        codes = rng.integers(0, 16, size=(64, 32)).astype(np.uint8)
        codes[:, 0] = rng.choice([6, 7, 14, 15], size=64)  # |v| in {4, 6} fixes the scale at 2**e
        vals = np.array([E2M1_TABLE[c & 7] for c in codes.reshape(-1)]).reshape(codes.shape)
        vals = np.where(codes & 8, -vals, vals) * 2.0 ** e
        packed, sc = mxfp4.encode(vals)
        assert (sc == e + 127).all(), e
        assert np.array_equal(mxfp4.unpack_nibbles(packed), codes), e


def test_roundtrip_every_code_many_scales():
    check_roundtrip()


def _bf16_values_up_to(limit):
    bits = np.arange(0, 0x8000, dtype=np.uint32)
    bits = bits[(bits >> 7) != 0xFF]          # drop inf/NaN patterns
    v = (bits << 16).view(np.float32).astype(np.float64)
    v = v[v <= limit]
    return np.concatenate([v, -v])


def _nearest_exact(q):
    """Nearest E2M1 magnitude code by exact rational distance; ties to even mantissa."""
    a = abs(Fraction(q))
    best = None
    for c, m in enumerate(E2M1_TABLE):
        d = abs(a - Fraction(m))
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def check_bf16_window():
    v = _bf16_values_up_to(4.0)
    blk = np.zeros((v.size, 32))
    blk[:, 0] = 4.0      # amax = 4 -> X = 1 for every row
    blk[:, 1] = v
    packed, sc = mxfp4.encode(blk)
    assert (sc == 127).all()
    got = mxfp4.unpack_nibbles(packed)[:, 1]
    # every value against exact rational rounding
    cache = {}
    for i in range(v.size):
        a = abs(v[i])
        if a not in cache:
            cache[a] = _nearest_exact(a)
        want = cache[a] | (8 if np.signbit(v[i]) else 0)
        assert got[i] == want, (v[i], got[i], want)


def test_exhaustive_bf16_one_window():
    check_bf16_window()


def test_zero_block_and_sign():
    blk = np.zeros((2, 32))
    blk[1, 3] = -0.0
    packed, sc = mxfp4.encode(blk)
    assert (packed == 0).all() and (sc == 0).all()


def test_packer_equals_oracle_encoder_random():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[3, :32] = 0
    w[5, 40] = 1e-30
    p1, s1 = fixtures.pack_mxfp4_rows(w)
    p2, s2 = mxfp4.encode(w.astype(np.float64))
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
