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


def encode(x):
    """float array -> uint8 codes: RNE to the nearest E4M3FN value, saturating.

    NaN inputs encode to 0x7F (with the input's sign bit).  Vectorised over
    the array, one comparison per step:
      1. a = |x|; values at or above 448 take code 0x7E;
      2. hi = first non-negative code whose value is >= a, lo = hi - 1;
      3. pick the nearer of lo / hi, ties to the even code;
      4. put the sign bit back.
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a_clean = np.where(nan, 0.0, a)
    sat = a_clean >= MAX_FINITE
    a_in = np.where(sat, 0.0, a_clean)
    hi = np.searchsorted(_POS_VALUES, a_in, side="left")  # 0..0x7E
    exact = _POS_VALUES[hi] == a_in
    lo = np.maximum(hi - 1, 0)
    d_lo = a_in - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a_in
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & 1) == 1))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo))
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def quantize_f32(x_f32, scale_f32):
    """Codes for x / scale, the division done in IEEE float32 (as stored data
    is: both operands are float32 and the quotient is rounded once), then
    encoded by ``encode``."""
    q = np.asarray(x_f32, dtype=np.float32) / np.asarray(scale_f32, dtype=np.float32)
    return encode(q.astype(np.float64))
