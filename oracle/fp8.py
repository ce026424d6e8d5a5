"""Oracle FP8 E4M3FN codec (test infrastructure only).

Mixed-precision KV storage is one of the features the PagedAttention blog
article lists (section 2.3, new features); the storage format used here is
the OCP 8-bit E4M3 "FN" format, written from its definition:

* bit 7 sign, bits 6..3 exponent with bias 7, bits 2..0 mantissa;
* exponent field 0 encodes subnormals: (-1)^s * 2^-6 * m/8;
* exponent field e in 1..15 encodes (-1)^s * 2^(e-7) * (1 + m/8),
  except e = 15, m = 7 (codes 0x7F and 0xFF), which are NaN;
* no infinities; the largest finite magnitude is 2^8 * 1.75 = 448.

Encoding is round-to-nearest, ties to the code with an even mantissa,
saturating to +-448 (the reading used for storing K/V: scales are chosen so
that the block's amax maps to 448, and nothing may become NaN).  The sign of
the input is kept, so small negative values round to -0 (code 0x80).
"""
import numpy as np

MAX_FINITE = 448.0


def _decode_code(code):
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


def decode_table():
    """float64 value of each of the 256 codes (NaN for 0x7F / 0xFF)."""
    return np.array([_decode_code(c) for c in range(256)], dtype=np.float64)


_TABLE = decode_table()
# Non-negative finite codes 0x00..0x7E are increasing in value.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = _TABLE[:0x7F]


def decode(codes):
    """uint8 array of codes -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# Midpoints between neighbouring non-negative codes (exact in float64: each
# is a value of the format with one more mantissa bit).
_MIDPOINTS = (_POS_VALUES[:-1] + _POS_VALUES[1:]) / 2


def encode(x):
    """float array -> uint8 codes: RNE to the nearest E4M3FN value, saturating.

    NaN inputs encode to 0x7F (with the input's sign bit).  With a = |x|:
      1. the nearest non-negative code is the number of midpoints below a
         (codes are in increasing order of value, so a lies between the
         values of that code and the next, nearer to the former exactly when
         it is below their midpoint);
      2. a value exactly on a midpoint is a tie: it goes to the even code of
         the two (the count above gives the lower one);
      3. beyond the last midpoint the count is 0x7E, so anything at or above
         448 takes code 0x7E (saturation);
      4. the sign bit is put back.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    code = np.searchsorted(_MIDPOINTS, np.where(nan, 0.0, a), side="left")  # 0..0x7E
    on_mid = _MIDPOINTS[np.minimum(code, _MIDPOINTS.size - 1)] == a
    code = code + (on_mid & ((code & 1) == 1))
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def quantize_f32(x_f32, scale_f32):
    """Codes for x / scale, the division done in IEEE float32 (as stored data
    is: both operands are float32 and the quotient is rounded once), then
    encoded by ``encode``."""
    q = np.asarray(x_f32, dtype=np.float32) / np.asarray(scale_f32, dtype=np.float32)
    return encode(q.astype(np.float64))
