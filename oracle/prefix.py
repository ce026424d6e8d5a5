"""Oracle prefix index over token ids (test infrastructure only).

The DataWhale notes' RadixAttention section: prompts that share a prefix
reuse the KV cache of that prefix; a new prompt is matched against the cached
token sequences by longest common prefix (LCP), the matched part reuses the
cached blocks and only the unmatched suffix is computed; the notes' exercise
keeps the cached sequences as a flat list and takes the best LCP over it.  This
oracle is that flat list, in insertion order, tied to the oracle allocator:

* insert(seq, n): the first n tokens of a live sequence become an entry.  Its
  divergence point d is its LCP with the entries before it; the entry
  provides positions d .. n-1 and holds one reference on each of its blocks
  that covers one of them (block indices d // bs .. (n-1) // bs), so those
  blocks outlive the sequence.
* match(tokens): hit = the largest LCP with any entry.  Block j of a hit
  (j < ceil(hit / bs)) is taken from the earliest entry whose LCP with the
  prompt exceeds q = min((j+1) * bs, hit) - 1, the last hit position in that
  block: that entry holds the same tokens as the prompt up to q, so its block
  j holds the right rows for every hit position in it.
* alloc_prompt_cached(seq, tokens): a new sequence made of the hit's blocks
  (one reference each) with length hit, then an append of the rest: the slots
  of the uncached suffix, and a copy-on-write pair if the suffix starts inside
  a shared block.  All or nothing (OOM leaves everything unchanged).
* clear(): every entry's references released, entries in insertion order,
  each entry's blocks by index; a block reaching zero goes back to the free
  list.

Readings where the notes are silent: the match is at token granularity (a partly
filled last block is shared and copied on the first write, as the allocator's
copy-on-write does); a full hit leaves an empty suffix (a caller wanting the
last token recomputed matches one token fewer); ties between equal LCPs take
the earliest entry.
"""
from .allocator import OOMError, ceil_div


def lcp_len(a, b):
    """Length of the longest common prefix (the notes' _lcp_len)."""
    n = 0
    while n < len(a) and n < len(b) and a[n] == b[n]:
        n += 1
    return n


class OraclePrefixIndex:
    def __init__(self, alloc):
        self.alloc = alloc
        self.entries = []          # (tokens, table, referenced block ids in index order)

    def _best(self, tokens):
        return max((lcp_len(e[0], tokens) for e in self.entries), default=0)

    def match(self, tokens):
        return self._best(list(tokens))

    def hit_blocks(self, tokens, hit):
        bs = self.alloc.block_size
        out = []
        for j in range(ceil_div(hit, bs)):
            q = min((j + 1) * bs, hit) - 1
            for toks, table, _ in self.entries:
                if lcp_len(toks, tokens) > q:
                    out.append(table[j])
                    break
        return out

    def insert(self, seq_id, tokens):
        tokens = [int(t) for t in tokens]
        a = self.alloc
        if seq_id not in a.tables:
            raise KeyError(seq_id)
        n = len(tokens)
        if n > a.lens[seq_id]:
            raise ValueError("more tokens than the sequence holds")
        d = self._best(tokens)
        table = list(a.tables[seq_id][:ceil_div(n, a.block_size)])
        refs = []
        if d < n:
            for j in range(d // a.block_size, (n - 1) // a.block_size + 1):
                a.refcount[table[j]] += 1
                refs.append(table[j])
        self.entries.append((tokens, table, refs))
        return d

    def alloc_prompt_cached(self, seq_id, tokens):
        """Returns (hit, slots of the suffix, cow pair or None)."""
        tokens = [int(t) for t in tokens]
        a = self.alloc
        if seq_id in a.tables:
            raise ValueError("sequence already exists")
        n, bs = len(tokens), a.block_size
        hit = self._best(tokens)
        blocks = self.hit_blocks(tokens, hit)
        cow = n > hit and hit % bs != 0
        need = ceil_div(n, bs) - ceil_div(hit, bs) + (1 if cow else 0)
        if len(a.free) < need:
            a.oom_count += 1
            raise OOMError()
        for b in blocks:
            a.refcount[b] += 1
        a.tables[seq_id] = list(blocks)
        a.lens[seq_id] = hit
        slots, pair = a.append_tokens(seq_id, n - hit)
        return hit, slots, pair

    def clear(self):
        a = self.alloc
        for _, _, refs in self.entries:
            for b in refs:
                a.refcount[b] -= 1
                if a.refcount[b] == 0:
                    a.free.append(b)
        self.entries = []

    def referenced_blocks(self):
        return sum(len(e[2]) for e in self.entries)
