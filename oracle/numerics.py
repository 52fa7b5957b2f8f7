"""Number formats the oracle needs: bfloat16 rounding and OCP e4m3 decoding.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Both functions are written from the formats' definitions, not from any GPU code:

* bfloat16 keeps the float32 exponent range and 8 significant bits (7 stored
  plus the implicit one).  Rounding a real value to bfloat16 therefore means
  rounding its significand to 8 bits, ties to even.
* OCP FP8 E4M3 ("fn" variant): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 encodes subnormals m * 2**-9; the single
  pattern S.1111.111 is NaN; there are no infinities; the largest finite
  magnitude is 448.
"""
import numpy as np


def round_bf16(x):
    """Round fp64 values to the nearest bfloat16 value (ties to even), as fp64.

    Uses frexp: x = f * 2**e with 0.5 <= |f| < 1, so 256*f carries exactly
    the 8 significant bits bfloat16 keeps; np.rint rounds half to even.
    Values here are far from the float32 overflow/underflow limits, so the
    exponent range of bfloat16 never matters.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(f * 256.0) / 256.0, e)


def _e4m3_value(c):
    """Value of each E4M3 byte code in the int64 array c, by the format's
    definition (sign, biased exponent, mantissa; subnormals; NaN)."""
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = np.ldexp(man / 8.0, -6)
    val = sign * np.where(exp == 0, subnormal, normal)
    return np.where((exp == 0xF) & (man == 0x7), np.nan, val)


# the 256 possible codes decoded once; decoding an array is a lookup
_E4M3_VALUES = _e4m3_value(np.arange(256, dtype=np.int64))


def decode_e4m3(codes):
    """Decode OCP FP8 E4M3 byte codes (uint8 array) to fp64 values."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]
