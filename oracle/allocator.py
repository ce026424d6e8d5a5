"""Oracle block allocator (test infrastructure only).

Follows the block manager the pages describe:

* DataWhale "llm-algo-leetcode (5)" notes, vLLM PagedAttention,
  ``KVCacheManager`` exercise: the free list starts as block ids in order and
  blocks are taken from its front; a prompt of n tokens takes
  ceil(n / block_size) blocks, checked against the free count before any block
  is taken (error "OOM"); a decode step adds one token and takes one new block
  exactly when the new length leaves a remainder of 1 modulo the block size.
* The same notes, section 4, copy-on-write: sequences with a common prefix
  point at the same physical blocks; a new physical block is taken only when
  a sequence writes into a block it shares.
* vLLM course ch. 4, "Block management strategy" table and allocation flow:
  a per-request block table, a free list that freed blocks return to, and
  blocks returned when the request ends.

Readings where the pages are silent:

* The free list is FIFO: initial order is the caller's (default 0..N-1),
  allocation pops the front, freed blocks go to the back in table order.
* Out of memory changes no state (the notes' decode step bumps the length
  before raising; this oracle checks first).
* Growth for k appended tokens is ceil((L+k)/bs) - ceil(L/bs) new blocks,
  which for k = 1 is "one block iff L % bs == 0", the notes' rule
  (new length % bs == 1) for every bs >= 2.
* Copy-on-write: if the last block is partly filled (L % bs != 0) and shared
  (refcount > 1), the writer takes one fresh block *before* any growth
  blocks, records the (src, dst) pair for a whole-block copy, and drops its
  reference to src.
"""
from collections import deque


class OOMError(RuntimeError):
    """Raised when the free list cannot satisfy a request (message "OOM")."""

    def __init__(self):
        super().__init__("OOM")


def ceil_div(a, b):
    return -(-a // b)


class OracleAllocator:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks < 0 or block_size < 1:
            raise ValueError("bad allocator geometry")
        self.num_blocks = num_blocks
        self.block_size = block_size
        if free_order is None:
            free_order = range(num_blocks)
        free_order = [int(b) for b in free_order]
        if sorted(free_order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..N-1")
        self.free = deque(free_order)
        self.refcount = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        self.cow_copies = 0
        self.oom_count = 0
        # a prefix index with eviction (oracle/radix.py) registers itself here;
        # an allocation that would run out asks it to reclaim blocks first
        self.evictor = None

    def _short(self, demand):
        """True if the blocks an operation needs cannot be had.  demand(alloc)
        is that need in a given state: an eviction can lower it (a block that
        loses its index reference needs no copy any more), so the evictor
        re-evaluates it after each eviction."""
        if len(self.free) >= demand(self):
            return False
        return self.evictor is None or not self.evictor.reclaim(
            lambda a: len(a.free) >= demand(a))

    def _append_demand(self, seq_id, k, dropped=None):
        """Blocks an append of k tokens to seq_id needs now: growth, plus one
        for a copy when its last block is partly filled and still shared
        (dropped: references a batch's earlier copies take off blocks)."""
        table, L, bs = self.tables[seq_id], self.lens[seq_id], self.block_size
        refs = self.refcount[table[-1]] - (dropped or {}).get(table[-1], 0) if table else 0
        cow = k > 0 and L % bs != 0 and refs > 1
        return ceil_div(L + k, bs) - ceil_div(L, bs) + (1 if cow else 0), cow

    # -- helpers -----------------------------------------------------------
    def _take(self):
        b = self.free.popleft()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def slot(self, seq_id, pos):
        """Physical slot of logical position pos: block * bs + offset."""
        table = self.tables[seq_id]
        return table[pos // self.block_size] * self.block_size + pos % self.block_size

    def _slots(self, seq_id, start, stop):
        return [self.slot(seq_id, p) for p in range(start, stop)]

    # -- operations --------------------------------------------------------
    def alloc_prompt(self, seq_id, num_tokens):
        """Blocks for a prompt; returns the slots of its tokens."""
        if seq_id in self.tables:
            raise ValueError("sequence already exists")
        if num_tokens < 0:
            raise ValueError("negative length")
        need = ceil_div(num_tokens, self.block_size)
        if self._short(lambda a: need):
            self.oom_count += 1
            raise OOMError()
        self.tables[seq_id] = [self._take() for _ in range(need)]
        self.lens[seq_id] = num_tokens
        return self._slots(seq_id, 0, num_tokens)

    def append_tokens(self, seq_id, k=1):
        """Append k tokens; returns (slots, cow) with cow = (src, dst) or None."""
        if seq_id not in self.tables:
            raise KeyError(seq_id)
        if k < 0:
            raise ValueError("negative count")
        if self._short(lambda a: a._append_demand(seq_id, k)[0]):
            self.oom_count += 1
            raise OOMError()
        table = self.tables[seq_id]
        L = self.lens[seq_id]
        bs = self.block_size
        grow = ceil_div(L + k, bs) - ceil_div(L, bs)
        needs_cow = self._append_demand(seq_id, k)[1]
        cow = None
        if needs_cow:
            src = table[-1]
            dst = self._take()
            self.refcount[src] -= 1
            table[-1] = dst
            cow = (src, dst)
            self.cow_copies += 1
        for _ in range(grow):
            table.append(self._take())
        self.lens[seq_id] = L + k
        return self._slots(seq_id, L, L + k), cow

    def append_tokens_batch(self, seq_ids, k=1):
        """k tokens appended to each listed sequence in order, all or nothing:
        the whole demand is checked first (a copy made for an earlier
        sequence drops its reference, which a later sequence sharing that
        block sees).  Returns [(slots, cow) per sequence]."""
        seq_ids = list(seq_ids)
        if len(set(seq_ids)) != len(seq_ids):
            raise ValueError("sequence listed twice")
        for s in seq_ids:
            if s not in self.tables:
                raise KeyError(s)

        def demand(a):
            dropped, need = {}, 0
            for s in seq_ids:
                n, cow = a._append_demand(s, k, dropped)
                need += n
                if cow:
                    last = a.tables[s][-1]
                    dropped[last] = dropped.get(last, 0) + 1
            return need

        if self._short(demand):
            self.oom_count += 1
            raise OOMError()
        return [self.append_tokens(s, k) for s in seq_ids]

    def fork(self, parent_id, child_id):
        """Child shares every block of the parent (refcount + 1)."""
        if parent_id not in self.tables:
            raise KeyError(parent_id)
        if child_id in self.tables:
            raise ValueError("child already exists")
        table = list(self.tables[parent_id])
        for b in table:
            self.refcount[b] += 1
        self.tables[child_id] = table
        self.lens[child_id] = self.lens[parent_id]

    def free_seq(self, seq_id):
        """Drop one reference to each block; blocks reaching zero go back."""
        table = self.tables.pop(seq_id)
        del self.lens[seq_id]
        for b in table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)

    # -- views -------------------------------------------------------------
    def block_table(self, seq_id):
        return list(self.tables[seq_id])

    def seq_len(self, seq_id):
        return self.lens[seq_id]

    def num_free(self):
        return len(self.free)

    def padded_tables(self, seq_ids, max_blocks):
        """Tables of the given sequences, padded with -1 to max_blocks."""
        rows = []
        for s in seq_ids:
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
        return rows
