"""Number formats of NVFP4: E2M1 element codes and E4M3 block scales.

The pages name the format only ("NVFP4", release post "capy-flash v0.7.1",
section "What shipped"; forum repost, paragraph "What it's for": the engine
"was born for" NVIDIA's NVFP4).  The definitions used here are the public
ones:

  E2M1  4 bits: sign (bit 3), 2 exponent bits, 1 mantissa bit, bias 1.
        Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.  No inf/NaN.
  E4M3  8 bits, OCP "FN" variant: sign (bit 7), 4 exponent bits (bias 7),
        3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); 0x7F/0xFF are
        NaN; no infinities; largest finite 448 (0x7E).

Encoders round to nearest with ties to the even code and saturate at the
largest finite value (a reading: the pages give the formats, not their rounding).
Test infrastructure only.
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E4M3_MAX = 448.0
E4M3_MAX_CODE = 0x7E


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit code (fp64); bit 3 is the sign."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def e4m3_decode(codes) -> np.ndarray:
    """Value of each 8-bit E4M3FN code (fp64); NaN for 0x7F and 0xFF."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    sub = m / 8.0 * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    v = s * np.where(e == 0, sub, nrm)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


# Non-negative finite E4M3 values, indexed by code 0x00..0x7E (increasing).
E4M3_GRID = e4m3_decode(np.arange(E4M3_MAX_CODE + 1))


def round_to_grid_even(a, grid: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to each a >= 0 (grid increasing, grid[0]
    = 0).  Exact ties go to the even index; values beyond grid[-1] go to the
    last index (saturation).  Comparisons are exact: inputs are fp32 and grid
    points have few significant bits, so the fp64 differences are exact."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(grid, a, side="left")          # grid[hi-1] < a <= grid[hi]
    hi_c = np.minimum(hi, len(grid) - 1)
    lo_c = np.maximum(hi - 1, 0)
    d_lo = a - grid[lo_c]
    d_hi = grid[hi_c] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0))
    idx = np.where(pick_hi, hi_c, lo_c)
    idx = np.where(hi >= len(grid), len(grid) - 1, idx)  # beyond the last point
    idx = np.where(a <= 0, 0, idx)
    return idx.astype(np.int64)


def e2m1_encode_magnitude(a) -> np.ndarray:
    """3-bit magnitude code of a >= 0: nearest of {0,.5,1,1.5,2,3,4,6}, ties to
    the even code, saturating at 6 (code 7)."""
    return round_to_grid_even(a, E2M1_MAGNITUDES)


def e4m3_encode_nonneg(s) -> np.ndarray:
    """E4M3FN code of s >= 0: round to nearest, ties to even, subnormals kept,
    saturate-to-finite at 448 (never NaN)."""
    return round_to_grid_even(s, E4M3_GRID)


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact value of bf16 bit patterns."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(a) -> np.ndarray:
    """Round values to bf16, nearest with ties to even (via exact fp32 when the
    value is already fp32; otherwise round-to-odd into fp32 first so the second
    rounding is exact)."""
    a = np.asarray(a, dtype=np.float64)
    f = a.astype(np.float32)
    # round-to-odd fp64 -> fp32: if inexact, force the fp32 lsb to 1 toward |a|
    back = f.astype(np.float64)
    fb = f.view(np.uint32).copy()
    inexact = back != a
    # move f toward zero if it was rounded away from zero, then set the lsb
    away = np.abs(back) > np.abs(a)
    fb = np.where(inexact & away, fb - 1, fb)
    fb = np.where(inexact, fb | 1, fb).astype(np.uint32)
    bits = fb.astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + bias) >> 16).astype(np.uint16)
