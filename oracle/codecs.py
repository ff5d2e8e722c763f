"""Number formats used by the KV cache, written from their definitions.

* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits -- the top half of an
  IEEE binary32.  Encoding from binary32 rounds to nearest, ties to even.
* FP8 E4M3 in the OCP "fn" flavour (OCP 8-bit Floating Point Specification,
  E4M3): 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities, the single
  NaN pattern S.1111.111, largest finite 1.75 * 2^8 = 448, smallest normal 2^-6,
  subnormals m * 2^-9.  The pages ask for "the platform FP8 dtype"; the reading
  taken is this format, encoded round-to-nearest-even with saturation to +-448
  and the sign kept for values that round to zero.

Every routine works on whole NumPy arrays and decides ties exactly in float64.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------- bfloat16


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_encode(x) -> np.ndarray:
    """binary32 values -> bf16 bit patterns, round to nearest, ties to even.

    The two bf16 neighbours of x are its truncation toward zero and the next
    representable value away from zero; the nearer one wins and a tie goes to the
    neighbour whose last mantissa bit is 0.  Values that are already bf16 pass
    through unchanged.  NaN inputs are not expected (they map to a quiet NaN).
    """
    x32 = np.asarray(x, dtype=np.float32)
    u = x32.view(np.uint32)
    down = (u >> 16).astype(np.uint32)            # truncation: same sign, |down| <= |x|
    up = down + 1                                 # next pattern away from zero
    xd = x32.astype(np.float64)
    vd = ((down << 16).view(np.float32)).astype(np.float64)
    vu = ((up << 16).astype(np.uint32).view(np.float32)).astype(np.float64)
    dd = np.abs(xd - vd)
    du = np.abs(vu - xd)
    pick_up = (du < dd) | ((du == dd) & ((down & 1) == 1))
    out = np.where(pick_up, up, down).astype(np.uint32)
    out = np.where(np.isnan(x32), np.uint32(0x7FC0), out)
    return out.astype(np.uint16)


# --------------------------------------------------------------- FP8 E4M3fn

def _e4m3_code_values() -> np.ndarray:
    """Value of every code 0..255 from the field layout (NaN for S.1111.111)."""
    codes = np.arange(256)
    s = (codes >> 7) & 1
    e = (codes >> 3) & 0xF
    m = codes & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    val = np.where(s == 1, -mag, mag)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return val.astype(np.float64)


E4M3_VALUES = _e4m3_code_values()
E4M3_MAX = 448.0
# non-negative finite codes 0x00 .. 0x7E in increasing value
_POS_GRID = E4M3_VALUES[:0x7F]


def e4m3_decode(codes: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """uint8 codes -> float64 values times the per-tensor scale."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)] * float(scale)


def e4m3_encode_unit(y32: np.ndarray) -> np.ndarray:
    """binary32 values (already divided by the scale) -> E4M3fn codes.

    Nearest grid value, ties to the even code (last mantissa bit 0), magnitudes
    beyond 448 saturate to 448, the sign bit is copied from the input.
    """
    y = np.asarray(y32, dtype=np.float32).astype(np.float64)
    a = np.abs(y)
    hi = np.searchsorted(_POS_GRID, a, side="left")        # first grid value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    exact = _POS_GRID[hi] == a
    d_lo = a - _POS_GRID[lo]
    d_hi = _POS_GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    mag = np.where(exact, hi, np.where(pick_hi, hi, lo))
    mag = np.where(a >= E4M3_MAX, 0x7E, mag)
    sign = np.signbit(y).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8)


def e4m3_encode(x, scale: float) -> np.ndarray:
    """Quantise x with a per-tensor scale: code = E4M3(fl32(x / scale)).

    The division is carried out in binary32 (IEEE, correctly rounded), the
    precision the store kernel uses, so both sides take the same rounding
    decision on the same binary32 quotient.
    """
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return e4m3_encode_unit(q)
