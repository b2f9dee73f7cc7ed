"""MXFP4 (E2M1 values, E8M0 scale per 32) decode and encode -- oracle side.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name the format only ("native MXFP4" experts in the TideLM README's
profile table; colibri's `matmul_mxfp4` in the cluster page's engine list).
Its definition is the OCP Microscaling Formats v1.0 one:
  * an E2M1 code is sign | 2 exponent bits | 1 mantissa bit, exponent bias 1;
    exponent 0 is subnormal (value m/2), otherwise 2**(e-1) * (1 + m/2);
  * an E8M0 scale byte c means 2**(c - 127); c = 255 is NaN;
  * encoding a 32-block: X = 2**(floor(log2(amax)) - 2) clamped to the E8M0
    exponent range, each v/X rounded to the nearest E2M1 value with ties to
    the even mantissa, magnitudes above 6 saturating; an all-zero block gets
    scale byte 0 and zero codes.
Element 2i of a row sits in the low nibble of byte i.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def e2m1_value(code: int) -> float:
    """Real value of one 4-bit E2M1 code, from the bit fields."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


VALUE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(code: int) -> float:
    if code == 255:
        return float("nan")
    return 2.0 ** (int(code) - 127)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> codes uint8 [..., K] (low nibble first)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Packed codes [N, K/2] and scale bytes [N, K/32] -> float64 [N, K]."""
    codes = unpack_nibbles(packed)
    n, kdim = codes.shape
    vals = VALUE[codes]
    sc = np.asarray(scales, dtype=np.int64)
    mult = np.where(sc == 255, np.nan, np.ldexp(1.0, sc - 127))
    return (vals.reshape(n, kdim // BLOCK, BLOCK) * mult[..., None]).reshape(n, kdim)


# Grid of E2M1 magnitudes indexed by the 3-bit magnitude code.
_MAG = VALUE[:8]
_MANT_ODD = np.array([c & 1 for c in range(8)])


def _nearest_magnitude(a: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code to each a >= 0; ties to the even mantissa.

    Written as the definition: the distance to every grid point, the minimum,
    and among equally near points the one whose mantissa bit is 0.
    """
    d = np.abs(a[..., None] - _MAG)
    best = d.min(axis=-1, keepdims=True)
    near = d == best
    pref = np.where(near, _MANT_ODD, 2)
    return np.argmin(pref, axis=-1).astype(np.uint8)


def encode(v: np.ndarray, chunk_rows: int = 256) -> tuple[np.ndarray, np.ndarray]:
    """float64 rows [N, K] -> (packed codes uint8 [N, K/2], scale bytes uint8 [N, K/32])."""
    v = np.asarray(v, dtype=np.float64)
    n, kdim = v.shape
    assert kdim % BLOCK == 0
    packed = np.empty((n, kdim // 2), dtype=np.uint8)
    scales = np.empty((n, kdim // BLOCK), dtype=np.uint8)
    for r0 in range(0, n, chunk_rows):
        blk = v[r0:r0 + chunk_rows].reshape(-1, kdim // BLOCK, BLOCK)
        amax = np.abs(blk).max(axis=-1)
        mant, ex = np.frexp(amax)              # amax = mant * 2**ex, mant in [0.5, 1)
        floor_log2 = ex.astype(np.int64) - 1
        e = np.clip(floor_log2 - 2, -127, 127)
        q = np.ldexp(blk, (-e)[..., None])     # v / X, exact
        mag = _nearest_magnitude(np.abs(q))    # saturation: |q| < 8, nearest is <= 6
        sign = np.signbit(q).astype(np.uint8)
        code = (sign << 3) | mag
        zero = amax == 0
        code[zero] = 0
        sc = (e + 127).astype(np.uint8)
        sc[zero] = 0
        code = code.reshape(code.shape[0], kdim)
        packed[r0:r0 + chunk_rows] = code[:, 0::2] | (code[:, 1::2] << 4)
        scales[r0:r0 + chunk_rows] = sc
    return packed, scales


def quantise(v: np.ndarray) -> np.ndarray:
    """decode(encode(v)): the values the layer actually multiplies."""
    return decode(*encode(v))
