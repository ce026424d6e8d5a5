"""Pins of the oracle allocator with a block size per request (buddy arena).

* The size rule at its boundaries.
* A hand-worked split / merge sequence on a 128-token arena.
* Requests all at the largest size reduce to the fixed-size oracle allocator
  over the arena's 64-token blocks (a different formulation).
* Random operations over mixed sizes: free and live blocks tile the arena
  exactly, no two free buddies are left unmerged, OOM happens exactly when a
  unit-level bitmap has too few fully free aligned regions (computed without
  the free lists), a refused call changes nothing, and a row pool written
  through every slot (in each sequence's own view layout, two heads) gives
  every live sequence back its own tokens."""
import copy

import numpy as np
import pytest

from oracle.allocator import OOMError, OracleAllocator
from oracle.buddy import SIZES, OracleBuddyAllocator, order_of, size_for


def test_size_rule():
    cases = {0: 8, 1: 8, 255: 8, 256: 16, 511: 16, 512: 32, 1023: 32, 1024: 64, 131072: 64}
    assert {n: size_for(n) for n in cases} == cases
    with pytest.raises(ValueError):
        order_of(4)


def _lists(a):
    return [list(f) for f in a.free]


def test_hand_worked_splits_and_merges():
    a = OracleBuddyAllocator(128)                     # 16 units, two 64-token blocks
    assert _lists(a) == [[], [], [], [0, 8]]
    assert a.alloc_prompt("A", 5, 8) == (8, [0, 1, 2, 3, 4])
    assert _lists(a) == [[1], [2], [4], [8]]          # unit 0 split down: halves 4, 2, 1 freed
    assert a.alloc_prompt("B", 20, 16) == (16, list(range(16, 32)) + [32, 33, 34, 35])
    assert a.block_table("B") == [1, 2] and _lists(a) == [[1], [6], [], [8]]
    assert a.alloc_prompt("C", 64, 64)[1] == list(range(64, 128))
    assert _lists(a) == [[1], [6], [], []]
    before = copy.deepcopy((_lists(a), a.refcount, a.tables))
    with pytest.raises(OOMError):                     # 3 blocks of 16 wanted, 1 obtainable
        a.alloc_prompt("D", 40, 16)
    assert copy.deepcopy((_lists(a), a.refcount, a.tables)) == before
    a.free_seq("A")                                   # 0 merges with 1; 2 is B's
    assert _lists(a) == [[], [6, 0], [], []]
    a.free_seq("B")                                   # 2 + 0 -> 0 (order 2); 4 + 6 -> 4, + 0 -> 0
    assert _lists(a) == [[], [], [], [0]]
    a.free_seq("C")
    assert _lists(a) == [[], [], [], [0, 8]]


def test_the_size_rule_is_used_when_no_size_is_named():
    a = OracleBuddyAllocator(4096)
    assert a.alloc_prompt(0, 300)[0] == 16 and len(a.block_table(0)) == 19
    assert a.alloc_prompt(1, 1500)[0] == 64 and len(a.block_table(1)) == 24
    assert a.alloc_prompt(2, 7)[0] == 8
    a.append_tokens(2, 2000)                          # the size stays for life
    assert a.block_size(2) == 8 and len(a.block_table(2)) == ceil(2007, 8)


def ceil(a, b):
    return -(-a // b)


@pytest.mark.parametrize("seed", range(4))
def test_largest_size_only_is_the_fixed_size_allocator(seed):
    rng = np.random.default_rng(seed)
    n_top = 24
    order = rng.permutation(n_top)
    a, o = OracleBuddyAllocator(64 * n_top, order), OracleAllocator(n_top, 64, order)
    live, sid = [], 0
    for _ in range(300):
        op = rng.integers(0, 4)
        if op == 0 or not live:
            n = int(rng.integers(0, 300))
            try:
                want = o.alloc_prompt(sid, n)
            except OOMError:
                with pytest.raises(OOMError):
                    a.alloc_prompt(sid, n, 64)
                continue
            assert a.alloc_prompt(sid, n, 64) == (64, want)
            live.append(sid)
            sid += 1
        elif op == 1:
            s = live[rng.integers(0, len(live))]
            m = int(rng.integers(1, 90))
            try:
                want = o.append_tokens(s, m)
            except OOMError:
                with pytest.raises(OOMError):
                    a.append_tokens(s, m)
                continue
            assert a.append_tokens(s, m) == want
        elif op == 2:
            s = live[rng.integers(0, len(live))]
            a.fork(s, sid)
            o.fork(s, sid)
            live.append(sid)
            sid += 1
        else:
            s = live.pop(rng.integers(0, len(live)))
            a.free_seq(s)
            o.free_seq(s)
        assert [u >> 3 for u in a.free[3]] == list(o.free)
        assert not any(a.free[:3])
        for s in live:
            assert a.block_table(s) == o.block_table(s)


def _bitmap_regions(a, k):
    """Fully free aligned regions of 2^k units, from a unit-level bitmap."""
    used = np.zeros(a.units, bool)
    for addr in a.refcount:
        used[addr:addr + (1 << _order_at(a, addr))] = True
    w = 1 << k
    return int(sum(not used[i:i + w].any() for i in range(0, a.units, w)))


def _order_at(a, addr):
    for s, k in a.order.items():
        if any((b << k) == addr for b in a.tables[s]):
            return k
    raise AssertionError(f"unit {addr} allocated but in no table")


def _check_tiling(a):
    cover = np.zeros(a.units, int)
    for k, f in enumerate(a.free):
        for u in f:
            assert u % (1 << k) == 0
            cover[u:u + (1 << k)] += 1
            if k < len(SIZES) - 1:
                assert (u ^ (1 << k)) not in f, "free buddies left unmerged"
    for addr in a.refcount:
        cover[addr:addr + (1 << _order_at(a, addr))] += 1
    assert (cover == 1).all()
    refs = {}
    for s, k in a.order.items():
        for b in a.tables[s]:
            refs[b << k] = refs.get(b << k, 0) + 1
    assert refs == a.refcount


class RowPool:
    """Rows of the arena, addressed as in the view of each sequence's block
    size: block i, head h, offset o -> row ((i * H + h) * bs + o)."""
    H = 2

    def __init__(self, a):
        self.a, self.rows = a, {}

    def addr(self, bs, slot, h):
        return ((slot // bs) * self.H + h) * bs + slot % bs

    def write(self, seq, slots, toks):
        bs = self.a.block_size(seq)
        for s, t in zip(slots, toks):
            for h in range(self.H):
                self.rows[self.addr(bs, s, h)] = (t, h)

    def cow(self, seq, pair):
        if pair is None:
            return
        bs = self.a.block_size(seq)
        src, dst = pair
        for o in range(bs):
            for h in range(self.H):
                r = self.addr(bs, src * bs + o, h)
                if r in self.rows:
                    self.rows[self.addr(bs, dst * bs + o, h)] = self.rows[r]

    def gather(self, seq):
        bs = self.a.block_size(seq)
        out = []
        for p in range(self.a.seq_len(seq)):
            s = self.a.slot(seq, p)
            got = [self.rows.get(self.addr(bs, s, h)) for h in range(self.H)]
            assert got[0] is not None and got[1] == (got[0][0], 1)
            out.append(got[0][0])
        return out


@pytest.mark.parametrize("seed,arena", [(0, 512), (1, 1024), (2, 2048), (3, 640)])
def test_random_mixed_sizes(seed, arena):
    rng = np.random.default_rng(50 + seed)
    a = OracleBuddyAllocator(arena, rng.permutation(arena // 64))
    pool = RowPool(a)
    live, sid, ooms = {}, 0, 0
    for step in range(500):
        op = rng.integers(0, 5)
        before = copy.deepcopy((_lists(a), a.refcount, a.tables, a.lens))
        try:
            if op == 0 or not live:
                n = int(rng.integers(0, arena // 3))
                bs = None if rng.random() < 0.5 else int(rng.choice(SIZES))
                k = order_of(size_for(n) if bs is None else bs)
                fits = _bitmap_regions(a, k) >= ceil(n, SIZES[k])
                try:
                    got_bs, slots = a.alloc_prompt(sid, n, bs)
                except OOMError:
                    assert not fits
                    raise
                assert fits and got_bs == SIZES[k]
                toks = [int(t) for t in rng.integers(0, 1000, n)]
                pool.write(sid, slots, toks)
                live[sid] = toks
                sid += 1
            elif op == 1:
                s = list(live)[rng.integers(0, len(live))]
                m = int(rng.integers(1, 40))
                slots, pair = a.append_tokens(s, m)
                pool.cow(s, pair)
                toks = [int(t) for t in rng.integers(0, 1000, m)]
                pool.write(s, slots, toks)
                live[s] = live[s] + toks
            elif op == 2:
                s = list(live)[rng.integers(0, len(live))]
                a.fork(s, sid)
                live[sid] = list(live[s])
                sid += 1
            else:
                s = list(live)[rng.integers(0, len(live))]
                a.free_seq(s)
                del live[s]
        except OOMError:
            ooms += 1
            assert copy.deepcopy((_lists(a), a.refcount, a.tables, a.lens)) == before
        _check_tiling(a)
        for s, toks in live.items():
            assert pool.gather(s) == toks
    assert ooms > 0 and len({a.block_size(s) for s in live} | {8}) >= 1
    for s in list(live):
        a.free_seq(s)
    assert _lists(a)[:3] == [[], [], []] and sorted(a.free[3]) == list(range(0, a.units, 8))
