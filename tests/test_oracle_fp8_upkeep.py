"""Pins of the oracle's fp8 write with scale upkeep (a block's scale follows
the amax of the rows it holds; earlier rows are requantised when it grows).

The worked example's codes are derived by hand from the E4M3FN definition
(sign | 4-bit exponent, bias 7 | 3-bit mantissa): with scales that are powers
of two every quotient is exactly representable, so each code follows from
value = 2^(e-7) * (1 + m/8) alone."""
import numpy as np
import pytest

from oracle import cache as C
from oracle import fp8


def _pool(N=2, H=1, bs=4, D=4):
    return np.zeros((N, H, bs, D), dtype=np.uint8), np.zeros((N, H), dtype=np.float32)


def _write(codes, scales, slots, rows, bs=4):
    C.write_rows_fp8_upkeep(codes, np.asarray(rows, dtype=np.float32)[:, None, :], slots,
                            scales, bs)


def test_worked_example_by_hand():
    codes, scales = _pool()
    # row 0: amax 112 -> scale 1/4; x / (1/4) = 6, -12, 2, 448
    _write(codes, scales, [0], [[1.5, -3.0, 0.5, 112.0]])
    assert scales[0, 0] == 0.25
    assert list(codes[0, 0, 0]) == [0x4C, 0xD4, 0x40, 0x7E]   # 1.5*2^2, -1.5*2^3, 2^1, 1.75*2^8
    # row 1: amax 224 -> scale 1/2; row 0 requantised to 3, -6, 1, 224
    _write(codes, scales, [1], [[0.25, 0.0, -224.0, 1.0]])
    assert scales[0, 0] == 0.5
    assert list(codes[0, 0, 0]) == [0x44, 0xCC, 0x38, 0x76]   # 1.5*2, -1.5*4, 1, 1.75*2^7
    assert list(codes[0, 0, 1]) == [0x30, 0x00, 0xFE, 0x40]   # 2^-1, 0, -448, 2
    # row 2: amax 10 < 224 -> scale stays, rows 0 and 1 untouched
    _write(codes, scales, [2], [[0.125, -0.0, 10.0, 7.0]])
    assert scales[0, 0] == 0.5
    assert list(codes[0, 0, 0]) == [0x44, 0xCC, 0x38, 0x76]
    assert list(codes[0, 0, 2]) == [0x28, 0x80, 0x5A, 0x56]   # 2^-2, -0, 1.25*2^4, 1.75*2^3
    # a fresh block of zeros keeps scale 0 and signed zeros; growth keeps them zero
    _write(codes, scales, [4], [[0.0, -0.0, 0.0, 0.0]])
    assert scales[1, 0] == 0.0 and list(codes[1, 0, 0]) == [0x00, 0x80, 0x00, 0x00]
    _write(codes, scales, [5], [[0.0, 0.0, 0.0, 896.0]])
    assert scales[1, 0] == 2.0
    assert list(codes[1, 0, 0]) == [0x00, 0x80, 0x00, 0x00]
    assert list(codes[1, 0, 1]) == [0x00, 0x00, 0x00, 0x7E]


def test_one_run_on_a_fresh_block_is_the_plain_write_at_amax_over_448():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((6, 3, 16)) * rng.uniform(0.1, 50, (6, 3, 1))).astype(np.float32)
    slots = np.arange(8, 14)                       # block 1 rows 0..5 (bs 8)
    a, sa = np.zeros((4, 3, 8, 16), np.uint8), np.zeros((4, 3), np.float32)
    C.write_rows_fp8_upkeep(a, x, slots, sa, 8)
    want_scale = np.abs(x).max(axis=(0, 2)).astype(np.float32) / np.float32(448)
    assert np.array_equal(sa[1], want_scale)
    b, sb = np.zeros_like(a), np.zeros_like(sa)
    sb[1] = want_scale
    C.write_rows_fp8(b, x, slots, sb, 8)
    assert np.array_equal(a, b)


def test_scale_is_the_running_amax_and_dequantised_rows_stay_close():
    """Any split of a block's rows into successive calls: the final scale is
    amax(all rows) / 448 (float32 division is monotone), every code is finite,
    and each value is within one RNE step per quantisation it went through."""
    rng = np.random.default_rng(11)
    bs, H, D = 16, 2, 8
    for trial in range(20):
        x = (rng.standard_normal((bs, H, D)) * rng.uniform(0.01, 100, (bs, H, 1))).astype(np.float32)
        cuts = sorted(rng.choice(np.arange(1, bs), size=rng.integers(0, 6), replace=False))
        edges = [0, *cuts, bs]
        codes, scales = np.zeros((3, H, bs, D), np.uint8), np.zeros((3, H), np.float32)
        requant = np.zeros((bs, H), dtype=np.int64)
        prev = np.zeros(H, np.float32)
        for lo, hi in zip(edges[:-1], edges[1:]):
            C.write_rows_fp8_upkeep(codes, x[lo:hi], np.arange(bs + lo, bs + hi), scales, bs)
            grew = scales[1] > prev
            requant[:lo] += grew[None, :]
            prev = scales[1].copy()
        assert np.array_equal(scales[1], np.abs(x).max(axis=(0, 2)).astype(np.float32) / np.float32(448))
        deq = fp8.decode(codes[1]).transpose(1, 0, 2) * scales[1][None, :, None].astype(np.float64)
        assert np.all(np.isfinite(deq))
        step = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * scales[1][None, :, None]
        bound = (1 + requant[:, :, None]) * step * 1.001
        assert np.all(np.abs(deq - x) <= bound), trial


def test_smaller_rows_leave_the_block_alone():
    rng = np.random.default_rng(3)
    codes, scales = np.zeros((2, 2, 8, 4), np.uint8), np.zeros((2, 2), np.float32)
    big = rng.standard_normal((3, 2, 4)).astype(np.float32) * 10
    C.write_rows_fp8_upkeep(codes, big, [0, 1, 2], scales, 8)
    before, s0 = codes.copy(), scales.copy()
    C.write_rows_fp8_upkeep(codes, big * np.float32(0.5), [3, 4], scales, 8)
    assert np.array_equal(scales, s0)
    assert np.array_equal(codes[0, :, :3], before[0, :, :3])


def test_runs_and_the_one_run_per_block_contract():
    assert C.write_runs([5, 6, 7, 8, -1, 12, 13, 3], 4) == [
        (1, 1, [0, 1, 2]), (2, 0, [3]), (3, 0, [5, 6]), (0, 3, [7])]
    codes, scales = _pool(N=4)
    with pytest.raises(ValueError):
        _write(codes, scales, [4, -1, 5], [[1, 1, 1, 1]] * 3)


def test_a_fresh_block_ignores_the_scale_its_previous_owner_left():
    """A run that starts a block (position 0) starts its scale from zero: the
    scale array still holds whatever the block's previous owner left."""
    codes, scales = _pool()
    scales[1, 0] = 100.0
    codes[1, 0] = 0x55
    _write(codes, scales, [4], [[1.5, -3.0, 0.5, 112.0]])
    assert scales[1, 0] == 0.25
    assert list(codes[1, 0, 0]) == [0x4C, 0xD4, 0x40, 0x7E]
