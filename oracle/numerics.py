"""Storage grids used by the layer, written from the number formats' definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bfloat16: the top 16 bits of an IEEE-754 binary32 value (1 sign bit,
  8 exponent bits, 7 stored significand bits), reached by
  round-to-nearest, ties-to-even on the dropped 16 bits.
* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 significand bits; no infinities; the all-ones code is NaN, so the
  largest finite magnitude is 1.75 * 2**8 = 448.  Normal values start at
  2**-6, subnormals are multiples of 2**-9.  Rounding is to nearest,
  ties to even, and saturates at +-448 (the reading taken for the
  pages' "FP8 scaling blocks" in [PB] "Roofline Validation", which fix
  neither the format nor the rounding).

All functions return float64 arrays holding values exactly on the grid.
"""

import numpy as np


def f32_round(a):
    """Round to IEEE binary32 (round-to-nearest-even) and return as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_round(a):
    """Round to bfloat16.

    The input is first taken as binary32 (every stored activation and
    weight in this layer starts life as a float32 value), then the low 16
    bits of its encoding are dropped with round-to-nearest, ties-to-even:
    add 0x7FFF plus the lowest kept bit, then truncate.  Infinities stay
    infinite; a finite value past the bf16 range becomes infinite, as in
    IEEE rounding.  NaN is not supported.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)) << np.uint64(16)
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


E4M3_MAX = 448.0
_E4M3_MIN_NORMAL_EXP = -6   # 2**-6 is the smallest normal magnitude
_E4M3_MANT_BITS = 3


def e4m3_round(a):
    """Round to the OCP E4M3 grid, nearest with ties to even, saturating at +-448.

    For |a| >= 2**-6 with binary exponent e (2**e <= |a| < 2**(e+1)) the
    grid spacing is 2**(e-3); below 2**-6 it is the subnormal spacing
    2**-9.  The quotient |a| / spacing is rounded half-to-even and scaled
    back, which also carries a value that rounds up into the next binade
    onto that binade's first grid point.  The sign is kept (so -0.0
    stays -0.0).
    """
    a = np.asarray(a, dtype=np.float64)
    mag = np.abs(a)
    # frexp: mag = m * 2**ex with m in [0.5, 1), so floor(log2(mag)) = ex - 1 (exactly).
    _, ex = np.frexp(np.maximum(mag, 2.0 ** _E4M3_MIN_NORMAL_EXP))
    spacing = np.ldexp(1.0, (ex - 1) - _E4M3_MANT_BITS)
    q = np.round(mag / spacing) * spacing          # np.round: half to even
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, a)


def e4m3_encode(q):
    """Encode values already on the E4M3 grid (finite, |q| <= 448) as uint8 codes."""
    q = np.asarray(q, dtype=np.float64)
    sign = np.signbit(q).astype(np.uint8) << np.uint8(7)
    mag = np.abs(q)
    m, ex = np.frexp(mag)                          # mag = m * 2**ex, m in [0.5, 1)
    biased = (ex - 1) + 7
    normal = mag >= 2.0 ** _E4M3_MIN_NORMAL_EXP
    # normal: mag = (1 + f/8) * 2**(biased-7), f in 0..7
    frac_normal = np.where(normal, np.round((2.0 * m - 1.0) * 8.0), 0.0)
    # subnormal (and zero): mag = f * 2**-9
    frac_sub = np.round(mag / 2.0 ** -9)
    exp_field = np.where(normal, biased, 0).astype(np.uint8)
    frac = np.where(normal, frac_normal, frac_sub).astype(np.uint8)
    return (sign | (exp_field << np.uint8(3)) | frac).astype(np.uint8)


def e4m3_decode(codes):
    """Decode uint8 E4M3 codes to float64 (the NaN code 0x7F/0xFF decodes to NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 0x7
    val = np.where(e == 0, f * 2.0 ** -9, (1.0 + f / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 0xF) & (f == 0x7), np.nan, val)
    return sign * val
