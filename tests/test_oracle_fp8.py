"""Pins for the oracle E4M3FN codec: an independent library and exhaustive checks."""
import numpy as np
import torch

from oracle import fp8


def test_decode_table_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    mine = fp8.decode_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_format_facts():
    t = fp8.decode_table()
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0          # largest finite
    assert t[0x01] == 2.0 ** -9                             # smallest subnormal
    assert t[0x08] == 2.0 ** -6                             # smallest normal
    assert t[0x38] == 1.0                                   # exponent 7 = bias
    assert np.all(np.diff(t[:0x7F]) > 0)


def test_round_trip_every_finite_code():
    t = fp8.decode_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    vals = t[codes]
    back = fp8.encode(vals)
    assert np.array_equal(back, codes)                      # includes -0 -> 0x80


def test_encode_matches_torch_in_range():
    """torch's float32 -> e4m3fn cast is round-to-nearest-even; inside the
    finite range it must agree with the oracle bit for bit."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 50,
        rng.standard_normal(20000).astype(np.float32) * 0.01,
        rng.uniform(-447.9, 447.9, 20000).astype(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.encode(x.astype(np.float64)), ref)


def test_ties_go_to_even_and_saturation():
    t = fp8.decode_table()
    pos = t[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2                          # exact in float64
    got = fp8.encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect.astype(np.uint8))
    assert np.array_equal(fp8.encode(np.array([448.0, 460.0, 464.0, 1e6, -1e6])),
                          np.array([0x7E, 0x7E, 0x7E, 0x7E, 0xFE], dtype=np.uint8))


def test_quantize_divides_in_float32():
    """A worked case where the precision of the division decides the code.

    x = 0x3CD9999A (0.026562500745...) and scale = 0.1f (0.100000001490...):
    the exact quotient is 0.26562500298..., just above the midpoint 0.265625
    between 0.25 (2^-2: exponent field 5, mantissa 0 -> code 0x28) and
    0.28125 (2^-2 * 1.125 -> code 0x29), so it rounds up to 0x29.  Rounded
    to float32 first, the quotient is exactly 0.265625, a tie, which goes
    to the even code 0x28.  Stored data divides in float32, so 0x28."""
    from fractions import Fraction
    x = np.array([0x3CD9999A], dtype=np.uint32).view(np.float32)
    s = np.float32(0.1)
    exact = Fraction(float(x[0])) / Fraction(float(s))
    assert Fraction(0.265625) < exact < Fraction(0.265625) + Fraction(1, 10**8)
    assert fp8.quantize_f32(x, s)[0] == 0x28
    assert fp8.encode(np.array([float(exact)]))[0] == 0x29      # the float64 quotient
    assert fp8.quantize_f32(-x, s)[0] == 0xA8                    # sign bit only
