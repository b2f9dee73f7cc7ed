"""MXFP6 (E2M3 values, E8M0 scale per 32) decode and encode -- oracle side.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The activation-format variant of the layer: the pages fix only the weights'
format (MXFP4), so the activation format is a reading; MXFP6 is the OCP
Microscaling Formats v1.0 "FP6 E2M3" element with the same E8M0 block scale:
  * an E2M3 code is sign | 2 exponent bits | 3 mantissa bits, exponent bias 1;
    exponent 0 is subnormal (value m/8), otherwise 2**(e-1) * (1 + m/8); the
    largest magnitude is 7.5 and there is no infinity or NaN;
  * encoding a 32-block: X = 2**(floor(log2(amax)) - 2) (2 = the exponent of
    E2M3's largest normal) clamped to the E8M0 exponent range, each v/X
    rounded to the nearest E2M3 value with ties to the even mantissa,
    magnitudes above 7.5 saturating; an all-zero block gets scale byte 0 and
    zero codes.
Layout of a row of K elements: K/32 blocks of 24 code bytes, element i of a
block at bits [6i, 6i + 6) of those bytes read as one little-endian 192-bit
number; then the K/32 scale bytes.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
BLOCK_BYTES = 24   # 32 six-bit codes


def e2m3_value(code: int) -> float:
    """Real value of one 6-bit E2M3 code, from the bit fields."""
    s = (code >> 5) & 1
    e = (code >> 3) & 3
    m = code & 7
    mag = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0)
    return -mag if s else mag


VALUE = np.array([e2m3_value(c) for c in range(64)], dtype=np.float64)


def row_bytes(K: int) -> int:
    """Bytes of one MXFP6 row of K elements (codes, then scales)."""
    return K // BLOCK * BLOCK_BYTES + K // BLOCK


def pack(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [N, K] (values 0..63) -> packed uint8 [N, 3K/4]."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, kdim = codes.shape
    blocks = codes.reshape(n, kdim // BLOCK, BLOCK).astype(np.uint64)
    out = np.zeros((n, kdim // BLOCK, BLOCK_BYTES), dtype=np.uint8)
    for i in range(BLOCK):                      # element i -> bits [6i, 6i + 6)
        bit = 6 * i
        for j in range(6):
            b = bit + j
            out[:, :, b // 8] |= (((blocks[:, :, i] >> j) & 1) << (b % 8)).astype(np.uint8)
    return out.reshape(n, kdim // BLOCK * BLOCK_BYTES)


def unpack(packed: np.ndarray) -> np.ndarray:
    """packed uint8 [N, 3K/4] -> codes uint8 [N, K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, nbytes = packed.shape
    nblk = nbytes // BLOCK_BYTES
    by = packed.reshape(n, nblk, BLOCK_BYTES)
    codes = np.zeros((n, nblk, BLOCK), dtype=np.uint8)
    for i in range(BLOCK):
        bit = 6 * i
        for j in range(6):
            b = bit + j
            codes[:, :, i] |= ((by[:, :, b // 8] >> (b % 8)) & 1) << j
    return codes.reshape(n, nblk * BLOCK)


def decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed codes [N, 3K/4] and scale bytes [N, K/32] -> float64 [N, K]."""
    codes = unpack(packed)
    n, kdim = codes.shape
    vals = VALUE[codes]
    sc = np.asarray(scales, dtype=np.int64)
    mult = np.where(sc == 255, np.nan, np.ldexp(1.0, sc - 127))
    return (vals.reshape(n, kdim // BLOCK, BLOCK) * mult[..., None]).reshape(n, kdim)


# Grid of E2M3 magnitudes indexed by the 5-bit magnitude code.
_MAG = VALUE[:32]
_MANT_ODD = np.array([c & 1 for c in range(32)])


def _nearest_magnitude(a: np.ndarray) -> np.ndarray:
    """Nearest E2M3 magnitude code to each a >= 0; ties to the even mantissa.

    Written as the definition: the distance to every grid point, the minimum,
    and among equally near points the one whose lowest mantissa bit is 0.
    """
    d = np.abs(a[..., None] - _MAG)
    best = d.min(axis=-1, keepdims=True)
    near = d == best
    pref = np.where(near, _MANT_ODD, 2)
    return np.argmin(pref, axis=-1).astype(np.uint8)


def encode(v: np.ndarray, chunk_rows: int = 64) -> tuple[np.ndarray, np.ndarray]:
    """float64 rows [N, K] -> (packed codes uint8 [N, 3K/4], scale bytes uint8 [N, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    n, kdim = v.shape
    assert kdim % BLOCK == 0
    codes = np.empty((n, kdim), dtype=np.uint8)
    scales = np.empty((n, kdim // BLOCK), dtype=np.uint8)
    for r0 in range(0, n, chunk_rows):
        blk = v[r0:r0 + chunk_rows].reshape(-1, kdim // BLOCK, BLOCK)
        amax = np.abs(blk).max(axis=-1)
        mant, ex = np.frexp(amax)              # amax = mant * 2**ex, mant in [0.5, 1)
        floor_log2 = ex.astype(np.int64) - 1
        e = np.clip(floor_log2 - 2, -127, 127)
        q = np.ldexp(blk, (-e)[..., None])     # v / X, exact
        mag = _nearest_magnitude(np.abs(q))    # |q| < 8: the nearest is at most 7.5
        sign = np.signbit(q).astype(np.uint8)
        code = (sign << 5) | mag
        zero = amax == 0
        code[zero] = 0
        sc = (e + 127).astype(np.uint8)
        sc[zero] = 0
        codes[r0:r0 + chunk_rows] = code.reshape(code.shape[0], kdim)
        scales[r0:r0 + chunk_rows] = sc
    return pack(codes), scales


def quantise(v: np.ndarray) -> np.ndarray:
    """decode(encode(v)): the values the layer actually multiplies."""
    return decode(*encode(v))
