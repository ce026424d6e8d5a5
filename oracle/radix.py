"""Oracle radix-tree prefix index with LRU eviction (test infrastructure only).

The DataWhale notes' RadixAttention section, step by step: cached token
sequences live in a radix tree (edges hold runs of tokens, nodes point at
the physical KV blocks); a new prompt is matched from the root; where a new
sequence leaves the middle of an edge the node is split into a common parent
and two children; when GPU memory is full the KV cache of leaf nodes is
deleted in least-recently-used order until there is room.

Block provenance is the flat-list oracle's (``oracle/prefix.py``): a node
remembers the entry that created its positions, an entry holds references on
its blocks from its divergence point on, block j of a hit comes from the
creator of the node holding position min((j+1) bs, h) - 1.  Without eviction
the two oracles must agree exactly (a pin of each by the other).

Readings for eviction, where the notes are silent:

* use: an insertion or a cached-prompt allocation stamps every node its walk
  entered with the operation's clock value (a split gives the new upper node
  the stamp of the node it came from); a plain match is a query and stamps
  nothing;
* a leaf (a node without children, not the root) is evicted whole, oldest
  stamp first, ties to the node created first; evicting it releases its
  creator's references on the blocks only it uses -- the block under its
  first position stays when the parent node has the same creator and shares
  it -- blocks reaching zero go back to the free list by index; its parent
  may become a leaf in turn;
* blocks of live sequences are never taken: eviction only drops the index's
  own references;
* automatic eviction is switched on per index (an allocator has at most
  one evicting index); then an allocation that would fail evicts leaves,
  oldest first, until its demand -- re-evaluated after every eviction,
  since dropping an index reference can make a copy-on-write unnecessary --
  fits the free list.  Whether that succeeds is decided on a dry run, so an
  allocation that still fails changes nothing (OOM keeps its all-or-nothing
  meaning); a cached-prompt allocation never evicts the nodes of its own
  hit;
* evict(min_free): explicit eviction, oldest leaves first, until the free
  list holds min_free blocks or no leaf is left.
"""
import copy

from .allocator import OOMError, ceil_div
from .prefix import lcp_len  # noqa: F401  (the same LCP definition)


class _Node:
    def __init__(self, nid, edge, start, creator, parent, stamp):
        self.id, self.edge, self.start = nid, list(edge), start
        self.creator, self.parent, self.stamp = creator, parent, stamp
        self.kids = {}
        self.alive = True

    @property
    def end(self):
        return self.start + len(self.edge)


class OracleRadixIndex:
    def __init__(self, alloc, auto_evict=False):
        self.alloc = alloc
        if auto_evict:
            if alloc.evictor is not None:
                raise ValueError("the allocator already has an evicting index")
            alloc.evictor = self
        self.clock = 0
        self.evicted = 0
        self._reset()

    def _reset(self):
        self.nodes = [_Node(0, [], 0, -1, -1, 0)]
        self.entries = []          # (table, {block index: block id}) per entry

    # -- walks ------------------------------------------------------------
    def _walk(self, tokens):
        """(depth, [(node, lo, hi)], stop node, offset in its edge)."""
        cur, depth, segs, stop, off = 0, 0, [], 0, 0
        n = len(tokens)
        while depth < n:
            k = self.nodes[cur].kids.get(tokens[depth])
            if k is None:
                break
            node = self.nodes[k]
            m = 0
            while m < len(node.edge) and depth + m < n and node.edge[m] == tokens[depth + m]:
                m += 1
            segs.append((k, depth, depth + m))
            depth += m
            stop, off = k, m
            if m < len(node.edge):
                return depth, segs, stop, off
            cur = k
        return depth, segs, stop, off

    def _stamp(self, segs):
        for k, _, _ in segs:
            self.nodes[k].stamp = self.clock

    def _hit_blocks(self, segs, h):
        bs, out, s = self.alloc.block_size, [], 0
        for j in range(ceil_div(h, bs)):
            q = min((j + 1) * bs, h) - 1
            while segs[s][2] <= q:
                s += 1
            out.append(self.entries[self.nodes[segs[s][0]].creator][0][j])
        return out

    # -- operations -------------------------------------------------------
    def match(self, tokens):
        return self._walk([int(t) for t in tokens])[0]

    def insert(self, seq_id, tokens):
        tokens = [int(t) for t in tokens]
        a, bs = self.alloc, self.alloc.block_size
        if seq_id not in a.tables:
            raise KeyError(seq_id)
        n = len(tokens)
        if n > a.lens[seq_id]:
            raise ValueError("more tokens than the sequence holds")
        self.clock += 1
        d, segs, stop, off = self._walk(tokens)
        self._stamp(segs)
        eid = len(self.entries)
        table = list(a.tables[seq_id][:ceil_div(n, bs)])
        refs = {}
        if d < n:
            for j in range(d // bs, (n - 1) // bs + 1):
                refs[j] = table[j]
            parent = stop
            low = self.nodes[stop]
            if stop != 0 and off < len(low.edge):
                up = _Node(len(self.nodes), low.edge[:off], low.start, low.creator, low.parent,
                           low.stamp)
                self.nodes.append(up)
                self.nodes[low.parent].kids[low.edge[0]] = up.id
                up.kids[low.edge[off]] = low.id
                low.edge = low.edge[off:]
                low.start += off
                low.parent = up.id
                parent = up.id
            leaf = _Node(len(self.nodes), tokens[d:], d, eid, parent, self.clock)
            self.nodes.append(leaf)
            self.nodes[parent].kids[tokens[d]] = leaf.id
        for b in refs.values():
            a.refcount[b] += 1
        self.entries.append((table, refs))
        return d

    def alloc_prompt_cached(self, seq_id, tokens):
        tokens = [int(t) for t in tokens]
        a, bs = self.alloc, self.alloc.block_size
        if seq_id in a.tables:
            raise ValueError("sequence already exists")
        self.clock += 1
        n = len(tokens)
        h, segs, _, _ = self._walk(tokens)
        cow = n > h and h % bs != 0
        need = ceil_div(n, bs) - ceil_div(h, bs) + (1 if cow else 0)
        if len(a.free) < need and not (a.evictor is self and self.reclaim(
                lambda al: len(al.free) >= need, {k for k, _, _ in segs})):
            a.oom_count += 1
            raise OOMError()
        self._stamp(segs)
        blocks = self._hit_blocks(segs, h)
        for b in blocks:
            a.refcount[b] += 1
        a.tables[seq_id] = list(blocks)
        a.lens[seq_id] = h
        slots, pair = a.append_tokens(seq_id, n - h)
        return h, slots, pair

    # -- eviction ---------------------------------------------------------
    def _leaves(self, protected):
        return [nd for nd in self.nodes[1:]
                if nd.alive and not nd.kids and nd.id not in protected]

    def _evict(self, leaf):
        a, bs = self.alloc, self.alloc.block_size
        refs = self.entries[leaf.creator][1]
        par = self.nodes[leaf.parent]
        first = leaf.start // bs
        if leaf.start % bs != 0 and leaf.parent != 0 and par.creator == leaf.creator:
            first += 1
        for j in range(first, (leaf.end - 1) // bs + 1):
            b = refs.pop(j, None)
            if b is not None:
                a.refcount[b] -= 1
                if a.refcount[b] == 0:
                    a.free.append(b)
        del par.kids[leaf.edge[0]]
        leaf.alive = False

    def _evict_until(self, fits, protected):
        n = 0
        while not fits(self.alloc):
            cands = self._leaves(protected)
            if not cands:
                break
            self._evict(min(cands, key=lambda nd: (nd.stamp, nd.id)))
            n += 1
        self.evicted += n
        return n

    def reclaim(self, fits, protected=()):
        """Evict oldest leaves until fits(allocator) holds; False, with
        nothing changed, if evicting every unprotected leaf would not do."""
        trial = copy.deepcopy((self.alloc, self))[1]
        trial._evict_until(fits, set(protected))
        if not fits(trial.alloc):
            return False
        self._evict_until(fits, set(protected))
        return True

    def evict(self, min_free):
        """Evict oldest leaves until at least min_free blocks are free (or
        no leaf is left); returns how many leaves were evicted."""
        return self._evict_until(lambda a: len(a.free) >= min_free, set())

    def clear(self):
        a = self.alloc
        for _, refs in self.entries:
            for j in sorted(refs):
                b = refs[j]
                a.refcount[b] -= 1
                if a.refcount[b] == 0:
                    a.free.append(b)
        self._reset()

    def referenced_blocks(self):
        return sum(len(r) for _, r in self.entries)

    def live_nodes(self):
        return sum(1 for nd in self.nodes if nd.alive)
