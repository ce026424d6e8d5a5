"""Host model of prefill_kernel's V^T operand addressing (no GPU).

The kernel keeps V tiles row-major in LDS, 16-byte chunk c of row r stored at
chunk slot c ^ swz_v(r), and reads the MFMA A-operand V^T with gfx950's
transposing LDS read ds_read_b64_tr_b16.  Lane rule of that instruction (as
measured on the GPU): in each group of 16 lanes, lane i receives 16-bit
element i % 4 of the 8-byte pieces addressed by lanes i//4, i//4+4, i//4+8,
i//4+12, in that order.

For k-step tt, half p of the operand and dimension block db, the kernel's
lane address is
    (16 tt + 8 p) * row_bytes + rl * row_bytes + 16 cl + 8 (lane % 2)
        + 64 * (db ^ (swz_v(rl) / 4)),
rl = 4 (lane // 32) + (lane % 16) // 4, cl = 2 ((lane // 16) % 2) + (lane % 4) // 2.
The MFMA needs lane l to hold, for its 8 contraction slots e, key
16 tt + 8 (e // 4) + 4 (l // 32) + e % 4 (the permuted order of P's registers)
of dimension 32 db + l % 32."""
import itertools

import pytest

BN = 32  # keys per tile


def swz_v(r, chunks):
    return 4 * ((r * chunks // 16) % (chunks // 4))


def lane_addr(lane, tt, p, db, D):
    row_bytes, chunks = 2 * D, D // 8
    rl = 4 * (lane // 32) + (lane % 16) // 4
    cl = 2 * ((lane // 16) % 2) + (lane % 4) // 2
    return ((16 * tt + 8 * p) * row_bytes + rl * row_bytes + 16 * cl + 8 * (lane % 2)
            + 64 * (db ^ (swz_v(rl, chunks) // 4)))


def tile_lds(D):
    """LDS byte offset -> (key row, dimension) after the swizzled DMA."""
    row_bytes, chunks = 2 * D, D // 8
    m = {}
    for r in range(BN):
        for slot in range(chunks):
            c = slot ^ swz_v(r, chunks)
            for e in range(8):
                m[r * row_bytes + 16 * slot + 2 * e] = (r, 8 * c + e)
    return m


def tr16(addrs, lds):
    """ds_read_b64_tr_b16 on a wave: the 4 (row, dim) elements each lane gets."""
    out = []
    for lane in range(64):
        g, i = 16 * (lane // 16), lane % 16
        out.append([lds[addrs[g + 4 * k + i // 4] + 2 * (i % 4)] for k in range(4)])
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_transposing_reads_give_the_mfma_operand(D):
    lds = tile_lds(D)
    for tt, db in itertools.product(range(2), range(D // 32)):
        got = [[] for _ in range(64)]
        for p in range(2):
            addrs = [lane_addr(l, tt, p, db, D) for l in range(64)]
            assert all(a % 8 == 0 and 0 <= a <= BN * 2 * D - 8 for a in addrs)
            for l, v in enumerate(tr16(addrs, lds)):
                got[l] += v
        for l in range(64):
            want = [(16 * tt + 8 * (e // 4) + 4 * (l // 32) + e % 4, 32 * db + l % 32)
                    for e in range(8)]
            assert got[l] == want, (tt, db, l)


@pytest.mark.parametrize("D", [64, 128])
def test_transposing_reads_are_bank_conflict_free(D):
    """Each half-wave's 32 x 8 bytes hit all 64 four-byte banks once."""
    for tt, p, db in itertools.product(range(2), range(2), range(D // 32)):
        for half in (0, 1):
            banks = [((lane_addr(l, tt, p, db, D) + 4 * w) // 4) % 64
                     for l in range(32 * half, 32 * half + 32) for w in range(2)]
            assert len(set(banks)) == 64, (D, tt, p, db, half)


def test_a_wrong_swizzle_is_caught():
    """Without the swizzle term the model reports collisions (the check has teeth)."""
    D = 128

    def addr_noswz(lane):
        rl = 4 * (lane // 32) + (lane % 16) // 4
        cl = 2 * ((lane // 16) % 2) + (lane % 4) // 2
        return rl * 2 * D + 16 * cl + 8 * (lane % 2)
    banks = [((addr_noswz(l) + 4 * w) // 4) % 64 for l in range(32) for w in range(2)]
    assert len(set(banks)) < 64
