"""Oracle allocator with a block size per request (test infrastructure only).

The first page's "3.0" feature list: the page (block) size is adjusted to the
request's length, blocks of different sizes serve requests of different
lengths, to use memory better.  Readings where the page is silent:

* sizes: 8, 16, 32 and 64 tokens.  Memory is one arena of 8-token units; a
  block of 8 * 2^k tokens (order k) is 2^k consecutive units starting at a
  multiple of 2^k (a binary buddy system, the textbook way to carve one
  arena into power-of-two sizes).  In the view of the arena with block size
  b, block id i is units [i * b/8, (i+1) * b/8); slot = id * b + offset, as
  for any pool of block size b.
* size rule: the largest size b with b <= n / 16 (at least 8), n the
  request's length at allocation: a request starts with about 16 or more
  blocks, so its unused tail (under one block) is below 1/16 of it; longer
  requests get larger blocks (fewer table entries).  A caller may also name
  the size.  A sequence keeps its size for life (its table is in one view).
* free lists: one FIFO per order; the arena starts as its 64-token blocks in
  the caller's order (default ascending).  A request for order k takes the
  front of list k; if that list is empty it takes the front of the nearest
  larger non-empty list and splits it down, keeping the lower half and
  putting each upper half at the back of the list one order below.  A freed
  block merges with its buddy (the block at unit address a XOR 2^k) while
  the buddy is free at the same order, then goes to the back of its list.
* everything else is the fixed-size allocator's (oracle/allocator.py): all
  or nothing with the demand counted first (a request for m blocks of order
  k fits when the free lists can yield m of them: sum over j >= k of
  |list j| * 2^(j-k)), copy-on-write block taken before growth blocks,
  freed blocks returned in table order, reference counts per block.
"""
import copy
from collections import deque

from .allocator import OOMError, ceil_div

SIZES = (8, 16, 32, 64)
UNIT = SIZES[0]
TOP = len(SIZES) - 1           # order of the largest size
BLOCKS_PER_REQUEST = 16


def size_for(n):
    """Block size the size rule gives a request of n tokens."""
    b = UNIT
    for s in SIZES:
        if s * BLOCKS_PER_REQUEST <= n:
            b = s
    return b


def order_of(bs):
    if bs not in SIZES:
        raise ValueError(f"block size {bs} not in {SIZES}")
    return SIZES.index(bs)


class OracleBuddyAllocator:
    def __init__(self, arena_tokens, top_order=None):
        if arena_tokens <= 0 or arena_tokens % SIZES[-1]:
            raise ValueError("arena must be a positive multiple of the largest block size")
        self.units = arena_tokens // UNIT
        n_top = self.units >> TOP
        if top_order is None:
            top_order = range(n_top)
        top_order = [int(b) for b in top_order]
        if sorted(top_order) != list(range(n_top)):
            raise ValueError("top_order must be a permutation of the largest blocks")
        self.free = [deque() for _ in SIZES]
        self.free[TOP].extend(b << TOP for b in top_order)      # unit addresses
        self.refcount = {}                                       # unit address -> refs
        self.order = {}                                          # seq -> order
        self.tables = {}                                         # seq -> block ids in its view
        self.lens = {}
        self.cow_copies = 0
        self.oom_count = 0

    # -- buddy system --------------------------------------------------------
    def obtainable(self, k):
        return sum(len(self.free[j]) << (j - k) for j in range(k, TOP + 1))

    def _take(self, k):
        j = k
        while not self.free[j]:
            j += 1                    # callers check obtainable() first
        a = self.free[j].popleft()
        while j > k:
            j -= 1
            self.free[j].append(a + (1 << j))
        assert a not in self.refcount
        self.refcount[a] = 1
        return a

    def _give(self, a, k):
        del self.refcount[a]
        while k < TOP:
            buddy = a ^ (1 << k)
            if buddy not in self.free[k]:
                break
            self.free[k].remove(buddy)
            a = min(a, buddy)
            k += 1
        self.free[k].append(a)

    def _unit(self, seq, i):
        return self.tables[seq][i] << self.order[seq]

    # -- operations -----------------------------------------------------------
    def block_size(self, seq):
        return SIZES[self.order[seq]]

    def slot(self, seq, pos):
        bs = self.block_size(seq)
        return self.tables[seq][pos // bs] * bs + pos % bs

    def alloc_prompt(self, seq, n, bs=None):
        """Returns (block size, slots)."""
        if seq in self.tables:
            raise ValueError("sequence already exists")
        if n < 0:
            raise ValueError("negative length")
        bs = size_for(n) if bs is None else bs
        k = order_of(bs)
        need = ceil_div(n, bs)
        if self.obtainable(k) < need:
            self.oom_count += 1
            raise OOMError()
        self.order[seq] = k
        self.tables[seq] = [self._take(k) >> k for _ in range(need)]
        self.lens[seq] = n
        return bs, [self.slot(seq, p) for p in range(n)]

    def append_tokens(self, seq, m=1):
        """Returns (slots, cow (src id, dst id) in the sequence's view or None)."""
        if seq not in self.tables:
            raise KeyError(seq)
        if m < 0:
            raise ValueError("negative count")
        k, table, L = self.order[seq], self.tables[seq], self.lens[seq]
        bs = SIZES[k]
        cow = m > 0 and L % bs != 0 and self.refcount[table[-1] << k] > 1
        grow = ceil_div(L + m, bs) - ceil_div(L, bs)
        if self.obtainable(k) < grow + (1 if cow else 0):
            self.oom_count += 1
            raise OOMError()
        pair = None
        if cow:
            src = table[-1]
            dst = self._take(k) >> k
            self.refcount[src << k] -= 1
            table[-1] = dst
            pair = (src, dst)
            self.cow_copies += 1
        for _ in range(grow):
            table.append(self._take(k) >> k)
        self.lens[seq] = L + m
        return [self.slot(seq, p) for p in range(L, L + m)], pair

    def append_tokens_batch(self, seqs, m=1):
        """m tokens appended to each listed sequence in order, all or nothing
        (decided by running the whole batch on a copy first).  Returns
        [(slots, cow) per sequence]."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("sequence listed twice")
        for s in seqs:
            if s not in self.tables:
                raise KeyError(s)
        trial = copy.deepcopy(self)
        try:
            for s in seqs:
                trial.append_tokens(s, m)
        except OOMError:
            self.oom_count += 1
            raise
        return [self.append_tokens(s, m) for s in seqs]

    def fork(self, parent, child):
        if parent not in self.tables:
            raise KeyError(parent)
        if child in self.tables:
            raise ValueError("child already exists")
        k = self.order[parent]
        for b in self.tables[parent]:
            self.refcount[b << k] += 1
        self.order[child] = k
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]

    def free_seq(self, seq):
        k = self.order.pop(seq)
        table = self.tables.pop(seq)
        del self.lens[seq]
        for b in table:
            a = b << k
            self.refcount[a] -= 1
            if self.refcount[a] == 0:
                self._give(a, k)

    # -- views ----------------------------------------------------------------
    def block_table(self, seq):
        return list(self.tables[seq])

    def seq_len(self, seq):
        return self.lens[seq]

    def free_tokens(self):
        return sum(len(f) << j for j, f in enumerate(self.free)) * UNIT
