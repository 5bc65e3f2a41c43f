"""Number formats: bf16 inputs, FP4 E2M1 codes, FP8 E4M3 and E8M0 scales.

Oracle module (test infrastructure only; see the package docstring).

The pages name the formats only: the cache dtype ``nvfp4`` and the scale
modes of "BitDecoding-FP4 evaluation/config.py" (KV_MODES), and "one 1-byte
scale per 16-elem block" in the ``mem_ratio`` docstring of
"kv-landlords scripts/quant_ab.py". The bit-level definitions below are those
of the OCP 8-bit Floating Point specification (E4M3, "fn" flavour: no
infinities, S.1111.111 is NaN, max 448) and the OCP Microscaling Formats v1.0
specification (FP4 E2M1 elements, E8M0 shared scales).
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# bf16 (inputs are bf16 bit patterns held in uint16 arrays)
# --------------------------------------------------------------------------


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (bf16 is the top half)."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# FP4 E2M1 (OCP MX v1.0): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0
# --------------------------------------------------------------------------

#: magnitude of the 3-bit code m = (exp << 1) | mantissa, m = 0..7
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0


def e2m1_value(nibble) -> np.ndarray:
    """Value of a 4-bit E2M1 code (float64, exact)."""
    nib = np.asarray(nibble, dtype=np.uint8) & np.uint8(0xF)
    mag = E2M1_GRID[(nib & np.uint8(7)).astype(np.intp)]
    return np.where((nib >> np.uint8(3)) & np.uint8(1), -mag, mag)


def e2m1_encode(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """4-bit code of x relative to scale s: round |x|/s to the nearest point
    of the E2M1 grid, ties to the even code, saturating at 6.

    * The rounding is of the exact real ratio |x|/s. It is decided by exact
      comparisons of |x| with the midpoints between grid points times s; each
      such product has at most 27 significant bits (midpoints have at most 3,
      a float32 scale 24), so it is exact in float64.
    * "Ties to the even code": at a midpoint between codes m and m+1 the
      result is whichever of the two has mantissa bit 0.
    * The sign bit is the IEEE sign bit of x (so a negative x that rounds to
      magnitude 0 keeps its sign bit).
    * A zero scale encodes every element as the all-zero nibble.

    x: float32 array; s: float32 array broadcastable to x (non-negative).
    """
    x = np.asarray(x, dtype=np.float32)
    s = np.broadcast_to(np.asarray(s, dtype=np.float32), x.shape)
    ax = np.abs(x.astype(np.float64))
    s64 = s.astype(np.float64)
    code = np.zeros(x.shape, dtype=np.uint8)
    for m in range(7):
        mid = 0.5 * (E2M1_GRID[m] + E2M1_GRID[m + 1]) * s64
        above = ax > mid
        tie = ax == mid
        up_on_tie = (m + 1) % 2 == 0          # code m+1 is the even one
        code = code + (above | (tie & up_on_tie)).astype(np.uint8)
    sign = (x.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    nib = (sign << np.uint8(3)) | code
    return np.where(s64 == 0.0, np.uint8(0), nib).astype(np.uint8)


# --------------------------------------------------------------------------
# FP8 E4M3 ("fn": bias 7, no infinities, 0x7F/0xFF NaN, max 448)
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of an 8-bit E4M3 code (float64, exact; NaN for 0x7F/0xFF)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** (1 - 7), (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(sign == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


#: the 127 non-negative finite E4M3 values, by code 0x00..0x7E (increasing)
_E4M3_POS = e4m3_value(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Code of the E4M3 value nearest to v >= 0, ties to the even code,
    saturating: v above the largest finite value gives 448 (0x7E).

    Plain nearest-value search over the table of all non-negative finite
    codes; distances are exact in float64 (v is float32, table values have
    4 significant bits).
    """
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    if np.any(v < 0) or np.any(np.isnan(v)):
        raise ValueError("e4m3_encode takes non-negative finite scales")
    tab = _E4M3_POS
    hi = np.clip(np.searchsorted(tab, v, side="left"), 0, len(tab) - 1)
    lo = np.clip(hi - 1, 0, len(tab) - 1)
    d_lo = np.abs(v - tab[lo])
    d_hi = np.abs(tab[hi] - v)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(v >= E4M3_MAX, 0x7E, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# E8M0 (OCP MX v1.0 shared scale): 2**(code - 127), 0xFF NaN
# --------------------------------------------------------------------------


def e8m0_value(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))
