"""Number codecs for the oracle (test infrastructure only).

bf16: the top 16 bits of an IEEE-754 binary32; decoding is exact. Encoding
rounds a float64 to the nearest bf16, ties to even, in one step (no detour
through float32, which could round twice).

E4M3FN (the OCP 8-bit float with 4 exponent bits, bias 7, 3 mantissa bits, no
infinities, NaN at S.1111.111): the fp8 KV format of the pages' quantised
decode ("[Kernel][Perf] Optimize paged-attention metadata decode", ROCm/FlyDSL
PR #910, "Pull request overview": per-token / per-tensor KV quantisation
modes). gfx950 uses this OCP variant, not gfx942's FNUZ one.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16/int16 bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 value (as float64), ties to even.

    A bf16 normal number at binary exponent e (x = m * 2**e, 0.5 <= |m| < 1)
    has 8 significant bits, so its spacing is 2**(e - 8); below the smallest
    normal (2**-126) the spacing stays 2**-133. Scaling by a power of two is
    exact, and numpy.rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    ulp_exp = np.maximum(e, -125) - 8
    out[fin] = np.ldexp(np.rint(np.ldexp(x[fin], -ulp_exp)), ulp_exp)
    big = np.abs(out) > 3.3895313892515355e38  # largest finite bf16
    out[big] = np.copysign(np.inf, out[big])
    return out


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), round to nearest even."""
    r = round_to_bf16(x).astype(np.float32)  # exact: r is a bf16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def e4m3fn_to_f64(codes) -> np.ndarray:
    """E4M3FN bytes -> float64, from the format's definition.

    sign s = bit 7, exponent e = bits 6..3, mantissa m = bits 2..0:
      e == 15 and m == 7    NaN
      e == 0                (-1)**s * (m / 8) * 2**-6        (subnormal)
      otherwise             (-1)**s * (1 + m / 8) * 2**(e - 7)
    """
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _e4m3fn_nonneg_values() -> np.ndarray:
    """Values of the 127 non-negative finite codes 0x00 .. 0x7E, in code order
    (which is value order)."""
    return e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))


def e4m3fn_encode(x) -> np.ndarray:
    """Finite values with |x| <= 448 -> E4M3FN bytes, round to nearest, ties
    to even.

    The definition written out: the code whose value is nearest to x; when x
    lies exactly halfway between two neighbouring codes, the one with mantissa
    LSB 0 (codes are ordered by value, so that is the even code). The sign bit
    is set for x < 0 (and for -0.0).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > 448.0):
        raise ValueError("e4m3fn_encode takes finite values with |x| <= 448")
    vals = _e4m3fn_nonneg_values()
    a = np.abs(x)
    hi = np.searchsorted(vals, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == vals[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(x)
    return np.where(neg, code | 0x80, code).astype(np.uint8)
