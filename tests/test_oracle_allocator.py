"""Pins for the oracle allocator and gather against the pages and invariants."""
import copy
import json
import os

import numpy as np
import pytest

from oracle import cache as C
from oracle.allocator import OOMError, OracleAllocator, ceil_div

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kvcache_manager_cases.json")


def _cases():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


@pytest.mark.parametrize("name", ["prefill_decode_gather", "block_boundary"])
def test_worked_example_counts_and_gather(name):
    """The notes' exercise: block counts after prefill and decode, then the
    gathered cache of blocks filled with constants (values from the pages)."""
    c = _cases()[name]
    a = OracleAllocator(c["num_blocks"], c["block_size"])
    a.alloc_prompt(7, c["prompt_len"])
    assert len(a.block_table(7)) == c["after_prefill"]["table_len"]
    if "num_free" in c["after_prefill"]:
        assert a.num_free() == c["after_prefill"]["num_free"]
    for d in c["decodes"]:
        a.append_tokens(7, 1)
        assert a.seq_len(7) == d["seq_len"]
        assert len(a.block_table(7)) == d["table_len"]
        if "num_free" in d:
            assert a.num_free() == d["num_free"]
    # the exercise's pool has no head axis: use H = 1 in the [N, H, bs, D] layout
    pool = np.zeros((c["num_blocks"], 1, c["block_size"], c["head_dim"]), dtype=np.float32)
    for b, v in zip(a.block_table(7), c["fill_values"]):
        pool[b] = v
    g = C.to_float64(C.gather(pool.view(np.uint32), a.block_table(7), a.seq_len(7), c["block_size"]),
                     C.F32)[:, 0, :]
    assert list(g.shape) == c["gathered_shape"]
    for lo, hi, v in c["gathered_rows"]:
        assert np.all(g[lo:hi] == v)


def test_worked_example_oom():
    c = _cases()["oom"]
    a = OracleAllocator(c["num_blocks"], c["block_size"])
    with pytest.raises(RuntimeError) as e:
        a.alloc_prompt(3, c["prompt_len"])
    assert c["expect_error"] in str(e.value)
    assert a.num_free() == 1 and 3 not in a.tables


def _state(a):
    return (list(a.free), list(a.refcount), copy.deepcopy(a.tables), dict(a.lens))


def _check_invariants(a):
    bs = a.block_size
    used = set()
    total_refs = 0
    for s, t in a.tables.items():
        assert len(t) == ceil_div(a.lens[s], bs)
        used.update(t)
        total_refs += len(t)
    assert sum(a.refcount) == total_refs
    assert len(a.free) + len(used) == a.num_blocks
    assert not (set(a.free) & used)
    for b in range(a.num_blocks):
        assert (a.refcount[b] == 0) == (b not in used)


@pytest.mark.parametrize("bs", [2, 4, 16, 32])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_op_sequences_keep_invariants(bs, seed):
    """Random prompt / append / fork / free sequences: table length is always
    ceil(L / bs); a one-token append takes a new block exactly when the new
    length % bs == 1 (the notes' rule); OOM happens exactly when demand exceeds
    the free count and changes nothing."""
    rng = np.random.default_rng(seed)
    N = 40
    a = OracleAllocator(N, bs, rng.permutation(N))
    next_id = 0
    for _ in range(600):
        op = rng.integers(0, 5)
        live = list(a.tables)
        before = _state(a)
        try:
            if op == 0 or not live:
                n = int(rng.integers(0, 3 * bs + 2))
                need = ceil_div(n, bs)
                oom_expected = need > a.num_free()
                a.alloc_prompt(next_id, n)
                assert not oom_expected
                next_id += 1
            elif op == 1:
                s = live[int(rng.integers(len(live)))]
                L = a.seq_len(s)
                t_before = len(a.block_table(s))
                shared_partial = L % bs != 0 and a.refcount[a.block_table(s)[-1]] > 1
                demand = (1 if L % bs == 0 else 0) + (1 if shared_partial else 0)
                oom_expected = demand > a.num_free()
                _, cow = a.append_tokens(s, 1)
                assert not oom_expected
                grew = len(a.block_table(s)) - t_before
                assert grew == (1 if a.seq_len(s) % bs == 1 else 0)
                assert (cow is not None) == shared_partial
            elif op == 2:
                s = live[int(rng.integers(len(live)))]
                k = int(rng.integers(1, 2 * bs + 3))
                L = a.seq_len(s)
                demand = ceil_div(L + k, bs) - ceil_div(L, bs)
                if L % bs != 0 and a.refcount[a.block_table(s)[-1]] > 1:
                    demand += 1
                oom_expected = demand > a.num_free()
                a.append_tokens(s, k)
                assert not oom_expected
                assert a.seq_len(s) == L + k
            elif op == 3:
                s = live[int(rng.integers(len(live)))]
                a.fork(s, next_id)
                assert a.block_table(next_id) == a.block_table(s)
                next_id += 1
            else:
                s = live[int(rng.integers(len(live)))]
                t = a.block_table(s)
                freed = [b for b in t if a.refcount[b] == 1]
                tail = list(a.free)
                a.free_seq(s)
                assert list(a.free) == tail + freed
        except OOMError:
            assert oom_expected
            assert _state(a) == before
        _check_invariants(a)


def test_fifo_order_and_slot_mapping():
    """Blocks come from the front of the caller's order; slots are
    block * bs + offset for each logical position."""
    order = [5, 2, 7, 0, 1, 3, 4, 6]
    a = OracleAllocator(8, 4, order)
    slots = a.alloc_prompt(0, 6)
    assert a.block_table(0) == [5, 2]
    assert slots == [20, 21, 22, 23, 8, 9]
    slots, cow = a.append_tokens(0, 3)
    assert cow is None and a.block_table(0) == [5, 2, 7]
    assert slots == [10, 11, 28]
    a.free_seq(0)
    assert list(a.free) == [0, 1, 3, 4, 6, 5, 2, 7]


def test_copy_on_write_on_shared_partial_block():
    """Fork mid-block: the first writer copies the shared partial block into a
    fresh block; the parent keeps the original; a later write by the parent
    (now sole owner) is in place."""
    a = OracleAllocator(10, 4)
    a.alloc_prompt(0, 6)                     # blocks [0, 1], block 1 half full
    a.fork(0, 1)
    assert a.refcount[0] == 2 and a.refcount[1] == 2
    slots, cow = a.append_tokens(1, 1)
    assert cow == (1, 2)                     # fresh block is the free-list front
    assert a.block_table(1) == [0, 2] and a.block_table(0) == [0, 1]
    assert slots == [2 * 4 + 2]
    assert a.refcount[1] == 1 and a.refcount[2] == 1 and a.refcount[0] == 2
    slots, cow = a.append_tokens(0, 1)
    assert cow is None and slots == [1 * 4 + 2]
    # CoW block is taken before growth blocks
    a.fork(0, 2)
    slots, cow = a.append_tokens(2, 3)       # 7 -> 10 tokens: copy block 1, then grow
    assert cow == (1, 3) and a.block_table(2) == [0, 3, 4]
    assert slots == [3 * 4 + 3, 4 * 4 + 0, 4 * 4 + 1]


def test_cow_needing_a_block_when_none_free_is_oom():
    a = OracleAllocator(2, 4)
    a.alloc_prompt(0, 5)
    a.fork(0, 1)
    before = _state(a)
    with pytest.raises(OOMError):
        a.append_tokens(1, 1)
    assert _state(a) == before


def test_gather_equals_logical_sequence():
    """Rows written through slots come back in logical order, whatever the
    physical placement."""
    rng = np.random.default_rng(3)
    bs, H, D, N = 4, 2, 8, 12
    a = OracleAllocator(N, bs, rng.permutation(N))
    logical = {}
    pool = np.full((N, H, bs, D), 0xFFFFFFFF, dtype=np.uint32)
    for s, n in [(0, 7), (1, 3), (2, 9)]:
        slots = a.alloc_prompt(s, n)
        x = rng.standard_normal((n, H, D), dtype=np.float32).view(np.uint32)
        C.write_rows(pool, x, slots, bs)
        logical[s] = x
    for s, x in logical.items():
        g = C.gather(pool, a.block_table(s), a.seq_len(s), bs)
        assert np.array_equal(g, x)
