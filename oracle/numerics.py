"""Number formats the oracle needs: bfloat16 rounding, OCP e4m3 decoding and
encoding, and per-row e4m3 quantisation.

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


# the finite non-negative E4M3 values in code order (codes 0x00..0x7E are
# increasing; 0x7F is NaN)
_E4M3_POS = _E4M3_VALUES[:0x7F]


def encode_e4m3(v):
    """OCP FP8 E4M3 codes of real values: the nearest finite E4M3 value,
    ties to the even code (mantissa LSB 0), saturating at +-448 (reading
    R13); the sign bit is the sign of v (so -0.0 and negatives that round to
    zero give 0x80)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")      # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo)
    code = np.where(_E4M3_POS[hi] == a, hi, code)        # exact values
    sign = np.signbit(v)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize_rows_e4m3(x):
    """Per-row E4M3 quantisation of activations (reading R13), every step in
    fp32 as the definition states: a = max |x_row|; the row's scale s =
    a / 448 and its multiplier r = 448 / a (fp32 divisions; both 1 for an
    all-zero row); q = encode_e4m3(x * r) with x * r an fp32 product
    (clamped to +-448, which the encoding's saturation gives anyway).
    x: [rows, K] values exactly representable in fp32 (bf16 activations).
    Returns (codes uint8 [rows, K], scales float32 [rows])."""
    x32 = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x32), axis=1)
    pos = a > 0
    safe = np.where(pos, a, np.float32(1.0)).astype(np.float32)
    s = np.where(pos, safe / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    r = np.where(pos, np.float32(448.0) / safe, np.float32(1.0)).astype(np.float32)
    v = (x32 * r[:, None]).astype(np.float32)
    return encode_e4m3(np.clip(v, np.float32(-448.0), np.float32(448.0))), s


def kv_cache_values(rows):
    """The values attention reads from an E4M3 KV cache (reading R14) for
    cached rows [..., D] (bf16 K or V rows as the cache received them):
    each row quantised as quantize_rows_e4m3 does, then decoded as
    bf16(fp32(code value x scale)) -- the fp32 product rounded to the
    nearest bf16, ties to even."""
    rows = np.asarray(rows)
    shape = rows.shape
    flat = rows.reshape(-1, shape[-1])
    codes, scale = quantize_rows_e4m3(flat)
    prod = (decode_e4m3(codes).astype(np.float32) * scale[:, None]).astype(np.float32)
    return round_bf16(prod.astype(np.float64)).reshape(shape)
