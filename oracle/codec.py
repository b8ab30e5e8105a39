"""Bit-level number formats for the oracle (test infrastructure only).

FP8 here is OCP E4M3FN (reading: the pages say only "FP8"; the GB200 page,
section 方法实现细节 / method details, describes the GEMM library as built for
FP8; E4M3FN is the FP8 that gfx950 matrix cores consume and the one
DeepSeek-style block-scaled inference uses).

E4M3FN definition, written out:
  byte = s eeee mmm, exponent bias 7
  e > 0           : (-1)^s * 2^(e-7) * (1 + m/8)
  e = 0           : (-1)^s * 2^(-6) * (m/8)           (subnormal)
  e = 15, m = 7   : NaN  (0x7F / 0xFF); there is no infinity
  largest finite  : 0x7E = 448

Encoding (reading): saturate to [-448, 448] first, then round to nearest,
ties to even mantissa, including the subnormal range (spacing 2^-9).

bf16: IEEE-754 binary32 truncated to its upper 16 bits (8 significant bits);
rounding from wider values is round-to-nearest-even, overflow goes to +-inf.

All arithmetic is float64; every intermediate is an exact power-of-two
scaling or an integer, so nothing here is subject to float rounding except
the one np.rint that *is* the rounding step.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F
BF16_NAN_BITS = 0x7FC0


def e4m3_decode(codes):
    """Decode E4M3FN bytes to float64 values (format definition above)."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e > 0,
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)),
                   np.ldexp(m / 8.0, -6))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_round(v):
    """Round float64 values to the nearest E4M3FN value (saturating, RNE).

    Returns the rounded values as float64 (NaN stays NaN).  In a binade
    [2^(x-1), 2^x) the spacing of E4M3 values is 2^(x-4); below 2^-6 the
    subnormal spacing 2^-9 applies.  np.rint rounds half to even, which on
    the integer multiple-of-spacing grid is exactly "ties to even mantissa".
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    step = np.maximum(ex, -5) - 4            # log2 of the spacing
    q = np.rint(np.ldexp(a, -step))
    mag = np.ldexp(q, step)
    out = np.where(np.signbit(v), -mag, mag)
    return np.where(np.isnan(v), np.nan, out)


def e4m3_encode(v):
    """Encode float64 values as E4M3FN bytes (saturating, RNE)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(invalid="ignore"):
        return _e4m3_encode(v)


def _e4m3_encode(v):
    # With a = min(|v|, 448) in binade 2^(x-1) <= a < 2^x and b = max(x, -5)
    # (b = -5 covers the subnormals and the lowest normal binade, which share
    # spacing 2^-9), the rounded magnitude is q * 2^(b-4) with integer
    # q = rint(a * 2^(4-b)) in [0, 16].  Its code is 8*b + 40 + q: for b > -5
    # that is exponent field b+6 and mantissa q-8 (q = 16 carries into the
    # next exponent with mantissa 0); for b = -5 it is q itself, which is the
    # subnormal code for q < 8 and the normal code for q >= 8.
    a = np.minimum(np.abs(v), E4M3_MAX)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, a)
    _, ex = np.frexp(a)
    b = np.maximum(ex, -5)
    q = np.rint(np.ldexp(a, 4 - b)).astype(np.int64)
    mag_code = np.where(a == 0.0, 0, 8 * b.astype(np.int64) + 40 + q)
    code = (np.signbit(v).astype(np.int64) << 7) | mag_code
    code = np.where(nan, E4M3_NAN_CODE, code)
    return code.astype(np.uint8)


def bf16_round(v):
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 has 8 significant bits: in binade [2^(x-1), 2^x) the spacing is
    2^(x-8); the smallest normal binade starts at 2^-126 and subnormals keep
    spacing 2^-133.  Results at or beyond 2^128 overflow to infinity.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    finite = np.isfinite(a)
    af = np.where(finite, a, 0.0)
    _, ex = np.frexp(af)
    step = np.maximum(ex, -125) - 8
    mag = np.ldexp(np.rint(np.ldexp(af, -step)), step)
    mag = np.where(mag >= 2.0 ** 128, np.inf, mag)
    mag = np.where(finite, mag, a)
    out = np.where(np.signbit(v), -mag, mag)
    return np.where(np.isnan(v), np.nan, out)


def bf16_bits(v):
    """Round float64 values to bf16 and return their 16-bit patterns (uint16)."""
    r = bf16_round(v)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(r), np.uint16(BF16_NAN_BITS), bits).astype(np.uint16)


def bf16_decode(bits):
    """bf16 bit patterns (uint16) to float64 values (exact)."""
    b = np.asarray(bits).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)
