"""Pins of the oracle prefix index: the notes' worked cases, and a content
check -- a pool of token ids written through every slot the allocator hands
out (and copied by every copy-on-write) must give back, for a sequence built
from a cached prefix, exactly its own prompt."""
import json
import os

import numpy as np
import pytest

from oracle.allocator import OOMError, OracleAllocator
from oracle.prefix import OraclePrefixIndex, lcp_len

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "radix_cache_cases.json")


def test_the_notes_worked_cases():
    g = json.load(open(GOLDEN))
    for c in g["lcp"]:
        assert lcp_len(c["a"], c["b"]) == c["len"]
    for bs in (1, 2, 3, 4):
        a = OracleAllocator(64, bs)
        x = OraclePrefixIndex(a)
        for i, t in enumerate(g["inserted"]):
            a.alloc_prompt(i, len(t))
            x.insert(i, t)
        for k, c in enumerate(g["match"]):
            p = c["prompt"]
            hit = x.match(p)
            assert hit == c["hit"] and p[:hit] == c["prefix"] and p[hit:] == c["suffix"]
            got_hit, slots, _ = x.alloc_prompt_cached(100 + k, p)
            assert got_hit == c["hit"] and len(slots) == len(c["suffix"])


class TokenPool:
    """The 'KV' of a slot is the id of the token written there."""

    def __init__(self, alloc):
        self.a = alloc
        self.slot = {}

    def write(self, slots, tokens):
        for s, t in zip(slots, tokens):
            self.slot[s] = t

    def cow(self, pair):
        if pair is None:
            return
        bs = self.a.block_size
        src, dst = pair
        for o in range(bs):
            if src * bs + o in self.slot:
                self.slot[dst * bs + o] = self.slot[src * bs + o]

    def gather(self, seq):
        return [self.slot[self.a.slot(seq, p)] for p in range(self.a.seq_len(seq))]


def _check_refs(a, x):
    live = sum(len(t) for t in a.tables.values())
    assert sum(a.refcount) == live + x.referenced_blocks()
    assert a.num_free() + sum(1 for r in a.refcount if r > 0) == a.num_blocks


@pytest.mark.parametrize("bs", [1, 2, 4, 16])
def test_cached_prompts_gather_their_own_tokens(bs):
    rng = np.random.default_rng(bs)
    a = OracleAllocator(4096, bs, rng.permutation(4096))
    x = OraclePrefixIndex(a)
    pool = TokenPool(a)
    bases = [list(rng.integers(0, 3, size=rng.integers(1, 60))) for _ in range(6)]
    live, sid = {}, 0
    for step in range(150):
        op = rng.integers(0, 4)
        if op == 0 or not live:                      # a new prompt, perhaps sharing a base
            base = bases[rng.integers(0, len(bases))]
            p = base[:rng.integers(0, len(base) + 1)] + list(rng.integers(0, 3, size=rng.integers(0, 20)))
            if not p:
                p = [1]
            hit, slots, pair = x.alloc_prompt_cached(sid, p)
            assert hit == max((lcp_len(e[0], p) for e in x.entries), default=0)
            pool.cow(pair)
            pool.write(slots, p[hit:])
            assert pool.gather(sid) == p
            live[sid] = list(p)
            sid += 1
        elif op == 1:                                # cache a live sequence's prefix
            s = list(live)[rng.integers(0, len(live))]
            n = int(rng.integers(0, len(live[s]) + 1))
            x.insert(s, live[s][:n])
        elif op == 2:                                # decode a token
            s = list(live)[rng.integers(0, len(live))]
            t = int(rng.integers(0, 3))
            slots, pair = a.append_tokens(s, 1)
            pool.cow(pair)
            pool.write(slots, [t])
            live[s].append(t)
            assert pool.gather(s) == live[s]
        else:                                        # finish a sequence
            s = list(live)[rng.integers(0, len(live))]
            a.free_seq(s)
            del live[s]
        _check_refs(a, x)
        for s, toks in live.items():                  # nobody's rows were overwritten
            assert pool.gather(s) == toks
    for s in list(live):
        a.free_seq(s)
    x.clear()
    assert a.num_free() == a.num_blocks and not any(a.refcount)


def test_cached_prompt_is_all_or_nothing():
    a = OracleAllocator(5, 4)
    x = OraclePrefixIndex(a)
    a.alloc_prompt(0, 6)
    x.insert(0, [1, 2, 3, 4, 5, 6])
    a.free_seq(0)                                    # the index keeps both blocks
    assert a.num_free() == 3
    before = (list(a.free), list(a.refcount))
    with pytest.raises(OOMError):                    # hit 6, +1 copy, +4 growth > 3 free
        x.alloc_prompt_cached(1, [1, 2, 3, 4, 5, 6] + [0] * 14)
    assert (list(a.free), list(a.refcount)) == before and 1 not in a.tables
    hit, slots, pair = x.alloc_prompt_cached(1, [1, 2, 3, 4, 5, 6, 7])
    assert hit == 6 and pair is not None and len(slots) == 1


def test_a_fully_cached_reinsert_references_nothing():
    a = OracleAllocator(16, 4)
    x = OraclePrefixIndex(a)
    a.alloc_prompt(0, 7)
    x.insert(0, list(range(7)))
    a.fork(0, 1)
    assert x.insert(1, list(range(7))) == 7 and x.entries[-1][2] == []
    assert x.insert(1, list(range(3))) == 3
