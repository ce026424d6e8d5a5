"""Pins of the oracle radix tree with LRU leaf eviction.

* Without eviction it must agree, step for step, with the flat-list prefix
  oracle (a different formulation of the same hit and block rules).
* Hand-worked LRU cases: which leaf goes first, which blocks come back, and
  that a block under a split stays while the upper half still needs it.
* Invariants on random operation sequences in a pool small enough to run
  out: a token-id pool written through every slot must give every live
  sequence back its own tokens (eviction never takes a live block), the
  reference counts add up, a refused allocation changes nothing."""
import copy

import numpy as np
import pytest

from oracle.allocator import OOMError, OracleAllocator
from oracle.prefix import OraclePrefixIndex
from oracle.radix import OracleRadixIndex
from tests.test_oracle_prefix import TokenPool, _check_refs


def _state(a):
    return list(a.free), list(a.refcount), {s: list(t) for s, t in a.tables.items()}, dict(a.lens)


@pytest.mark.parametrize("bs,seed", [(1, 0), (2, 1), (3, 2), (4, 3), (16, 4)])
def test_agrees_with_the_flat_list_without_eviction(bs, seed):
    rng = np.random.default_rng(100 + seed)
    N = 2000
    order = rng.permutation(N)
    a1, a2 = OracleAllocator(N, bs, order), OracleAllocator(N, bs, order)
    flat, tree = OraclePrefixIndex(a1), OracleRadixIndex(a2)
    bases = [list(rng.integers(0, 3, size=rng.integers(1, 40))) for _ in range(5)]
    live, sid = {}, 0
    for step in range(400):
        op = rng.integers(0, 6)
        if op <= 1 or not live:
            base = bases[rng.integers(0, len(bases))]
            p = base[:rng.integers(0, len(base) + 1)] + list(rng.integers(0, 3, size=rng.integers(0, 10)))
            assert flat.match(p) == tree.match(p)
            assert flat.alloc_prompt_cached(sid, p) == tree.alloc_prompt_cached(sid, p)
            live[sid] = list(p)
            sid += 1
        elif op == 2:
            s = list(live)[rng.integers(0, len(live))]
            n = int(rng.integers(0, len(live[s]) + 1))
            assert flat.insert(s, live[s][:n]) == tree.insert(s, live[s][:n])
        elif op == 3:
            s = list(live)[rng.integers(0, len(live))]
            k = int(rng.integers(1, 4))
            assert a1.append_tokens(s, k) == a2.append_tokens(s, k)
            live[s] += list(rng.integers(0, 3, size=k))
        elif op == 4:
            s = list(live)[rng.integers(0, len(live))]
            a1.free_seq(s)
            a2.free_seq(s)
            del live[s]
        elif rng.random() < 0.1:
            flat.clear()
            tree.clear()
        assert _state(a1) == _state(a2)
        assert flat.referenced_blocks() == tree.referenced_blocks()


def _cache(a, x, sid, tokens):
    """A finished request whose tokens stay cached: allocate, insert, free."""
    a.alloc_prompt(sid, len(tokens))
    x.insert(sid, tokens)
    table = a.block_table(sid)
    a.free_seq(sid)
    return table


def test_least_recently_used_leaf_goes_first():
    a = OracleAllocator(8, 2)
    x = OracleRadixIndex(a, auto_evict=True)
    assert _cache(a, x, 0, [1, 2, 3, 4]) == [0, 1]
    assert _cache(a, x, 1, [5, 6, 7, 8]) == [2, 3]
    assert _cache(a, x, 2, [9, 9, 9, 9]) == [4, 5]
    assert list(a.free) == [6, 7]
    hit, slots, pair = x.alloc_prompt_cached(3, [1, 2, 3, 4, 0])     # uses the first entry
    assert (hit, slots, pair) == (4, [12], None) and list(a.free) == [7]
    # 3 blocks wanted, 1 free: the oldest leaf (5 6 7 8) goes, its blocks
    # return in index order behind the free block
    assert a.alloc_prompt(4, 6) == [14, 15, 4, 5, 6, 7]
    assert a.block_table(4) == [7, 2, 3] and x.evicted == 1
    assert x.match([5, 6]) == 0 and x.match([9, 9, 9]) == 3 and x.match([1, 2, 3, 4]) == 4
    a.free_seq(3)
    assert list(a.free) == [6]
    assert a.alloc_prompt(5, 4) == [12, 13, 8, 9]                     # next oldest: 9 9 9 9
    assert a.block_table(5) == [6, 4] and x.evicted == 2
    assert x.match([9]) == 0 and x.match([1, 2, 3, 4]) == 4


def test_block_under_a_split_stays_while_the_upper_half_needs_it():
    a = OracleAllocator(6, 4)
    x = OracleRadixIndex(a, auto_evict=True)
    assert _cache(a, x, 0, [1, 2, 3, 4, 5, 6]) == [0, 1]
    hit, slots, pair = x.alloc_prompt_cached(1, [1, 2, 3, 4, 5, 7, 7])
    assert hit == 5 and pair == (1, 2) and slots == [9, 10]
    assert x.insert(1, [1, 2, 3, 4, 5, 7, 7]) == 5                   # splits 1..6 after 5
    a.free_seq(1)
    assert list(a.free) == [3, 4, 5] and x.live_nodes() == 4
    # leaves: [6] (entry 0) and [7 7] (entry 1), same stamp; [6] is older.
    # Evicting [6] frees nothing: block 1 also holds position 4, which the
    # upper half [1..5] (entry 0) still provides.  Then [7 7] frees block 2.
    assert x.evict(4) == 2 and list(a.free) == [3, 4, 5, 2]
    assert x.match([1, 2, 3, 4, 5, 6]) == 5
    hit, slots, pair = x.alloc_prompt_cached(2, [1, 2, 3, 4, 5])
    assert (hit, len(slots), pair) == (5, 0, None) and a.block_table(2) == [0, 1]
    # evicting the last leaf drops the index's references; the live
    # sequence keeps both blocks
    assert x.evict(6) == 1 and list(a.free) == [3, 4, 5, 2]
    assert a.refcount[0] == a.refcount[1] == 1 and x.referenced_blocks() == 0


def test_a_cached_prompt_never_evicts_its_own_hit():
    a = OracleAllocator(4, 2)
    x = OracleRadixIndex(a, auto_evict=True)
    _cache(a, x, 0, [1, 2, 3, 4])
    before = _state(a)
    with pytest.raises(OOMError):                  # hit 4, 3 more blocks, 2 free
        x.alloc_prompt_cached(1, [1, 2, 3, 4, 5, 6, 7, 8, 9, 10])
    assert _state(a) == before and x.match([1, 2, 3, 4]) == 4 and x.evicted == 0
    with pytest.raises(OOMError):                  # without the hit it may go
        a.alloc_prompt(1, 9)
    assert a.alloc_prompt(1, 8) and x.evicted == 1 and x.match([1]) == 0


def test_a_refused_allocation_evicts_nothing():
    a = OracleAllocator(6, 2)
    x = OracleRadixIndex(a, auto_evict=True)
    _cache(a, x, 0, [1, 2, 3])
    a.alloc_prompt(1, 4)
    before = _state(a)
    with pytest.raises(OOMError):                  # 4 wanted, 2 free + 2 evictable
        a.alloc_prompt(2, 9)
    assert _state(a) == before and x.match([1, 2, 3]) == 3 and x.evicted == 0


def test_eviction_can_remove_a_copy_from_the_demand():
    """A live sequence whose last, partly filled block is also held by the
    index would copy it on its next write.  With no free block, evicting the
    entry leaves it the only holder: the append then needs no block."""
    a = OracleAllocator(2, 4)
    x = OracleRadixIndex(a, auto_evict=True)
    a.alloc_prompt(0, 6)
    x.insert(0, [1, 2, 3, 4, 5, 6])
    assert a.num_free() == 0 and a.refcount == [2, 2]
    assert a.append_tokens(0, 1) == ([6], None)
    assert x.evicted == 1 and a.refcount == [1, 1] and a.num_free() == 0
    # without eviction the same append is out of memory
    b = OracleAllocator(2, 4)
    y = OracleRadixIndex(b)
    b.alloc_prompt(0, 6)
    y.insert(0, [1, 2, 3, 4, 5, 6])
    with pytest.raises(OOMError):
        b.append_tokens(0, 1)


def test_batch_append_evicts_for_the_whole_batch():
    a = OracleAllocator(6, 2)
    x = OracleRadixIndex(a, auto_evict=True)
    _cache(a, x, 9, [7, 7, 7, 7])                  # 2 blocks cached
    a.alloc_prompt(0, 2)
    a.alloc_prompt(1, 2)
    assert a.num_free() == 2
    out = a.append_tokens_batch([0, 1], 3)
    assert [len(s) for s, _ in out] == [3, 3] and x.evicted == 1 and a.num_free() == 0
    with pytest.raises(OOMError):
        a.append_tokens_batch([0, 1], 2)
    with pytest.raises(ValueError):
        a.append_tokens_batch([0, 0], 1)


def test_only_one_evicting_index_per_allocator():
    a = OracleAllocator(4, 2)
    OracleRadixIndex(a, auto_evict=True)
    OracleRadixIndex(a)
    with pytest.raises(ValueError):
        OracleRadixIndex(a, auto_evict=True)


@pytest.mark.parametrize("bs,N,seed", [(1, 40, 0), (2, 24, 1), (4, 12, 2), (3, 16, 3), (8, 8, 4)])
def test_random_operations_under_memory_pressure(bs, N, seed):
    rng = np.random.default_rng(300 + seed)
    a = OracleAllocator(N, bs, rng.permutation(N))
    x = OracleRadixIndex(a, auto_evict=True)
    pool = TokenPool(a)
    bases = [list(rng.integers(0, 3, size=rng.integers(1, 3 * bs + 4))) for _ in range(4)]
    live, sid, ooms = {}, 0, 0
    for step in range(400):
        op = rng.integers(0, 7)
        before = copy.deepcopy((_state(a), [(n.alive, n.stamp, list(n.edge)) for n in x.nodes]))
        try:
            if op <= 1 or not live:
                base = bases[rng.integers(0, len(bases))]
                p = base[:rng.integers(0, len(base) + 1)] + list(rng.integers(0, 3, size=rng.integers(0, 2 * bs)))
                p = p or [1]
                want = x.match(p)
                hit, slots, pair = x.alloc_prompt_cached(sid, p)
                assert hit == want
                pool.cow(pair)
                pool.write(slots, p[hit:])
                live[sid] = list(p)
                sid += 1
            elif op == 2:
                s = list(live)[rng.integers(0, len(live))]
                x.insert(s, live[s][:rng.integers(0, len(live[s]) + 1)])
            elif op == 3:
                s = list(live)[rng.integers(0, len(live))]
                t = [int(v) for v in rng.integers(0, 3, size=rng.integers(1, 3))]
                slots, pair = a.append_tokens(s, len(t))
                pool.cow(pair)
                pool.write(slots, t)
                live[s] += t
            elif op == 4:
                ids = list(live)[:rng.integers(1, len(live) + 1)]
                t = int(rng.integers(0, 3))
                for s, (slots, pair) in zip(ids, a.append_tokens_batch(ids, 1)):
                    pool.cow(pair)
                    pool.write(slots, [t])
                    live[s].append(t)
            elif op == 5:
                s = list(live)[rng.integers(0, len(live))]
                a.free_seq(s)
                del live[s]
            else:
                x.evict(int(rng.integers(0, N + 1)))
        except OOMError:
            ooms += 1
            assert (_state(a), [(n.alive, n.stamp, list(n.edge)) for n in x.nodes]) == before
        _check_refs(a, x)
        for s, toks in live.items():
            assert pool.gather(s) == toks
    assert x.evicted > 0 and ooms > 0
    for s in list(live):
        a.free_seq(s)
    x.clear()
    assert a.num_free() == N and not any(a.refcount)
