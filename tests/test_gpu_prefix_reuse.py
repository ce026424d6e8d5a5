"""Prefill over a cached prefix: prompts that share the longest cached
prefix of earlier ones reuse its blocks through the prefix index (C++ and
oracle side by side, bit for bit), the partly shared block is copied on the
first write, and pa_prefill_chunk runs only on the uncached suffix -- its
output equals the oracle's attention of that suffix over the whole prompt's
K/V (the cached rows included)."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_166_amd as pa
from oracle import attention as A
from oracle import cache as C
from oracle.prefix import OraclePrefixIndex
from tests.gpu_util import TOL, Scenario, assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv,bs", [("bf16", 16), ("f16", 32), ("bf16", 4)])
def test_suffix_prefill_over_a_cached_prefix(kv, bs):
    H, D = 4, 128
    sc = Scenario(600, H, bs, D, kv, seed=200 + bs)
    x, ox = pa.PrefixIndex(sc.alloc), OraclePrefixIndex(sc.ora)
    rng = np.random.default_rng(bs)
    system = list(rng.integers(0, 1000, size=300))
    # two cached conversations under one system prompt
    for sid, tail in ((0, 40), (1, 77)):
        p = system + list(rng.integers(0, 1000, size=tail))
        sc.prompt(sid, len(p))
        assert x.insert(sid, p) == ox.insert(sid, p)
        sc.tokens = getattr(sc, "tokens", {})
        sc.tokens[sid] = p
    sc.alloc.free_seq(0)                     # the index keeps its blocks alive
    sc.ora.free_seq(0)
    sc.seqs.remove(0)
    prompts = [
        sc.tokens[0][:331] + list(rng.integers(0, 1000, size=60)),   # inside seq 0's tail
        system[:213] + list(rng.integers(0, 1000, size=90)),         # inside the system prompt
        sc.tokens[1] + list(rng.integers(0, 1000, size=5)),          # all of seq 1, then more
        list(rng.integers(1000, 2000, size=33)),                      # nothing cached
    ]
    seqs, suffix = [], []
    for k, p in enumerate(prompts):
        sid = 10 + k
        hit, slots, pair = x.alloc_prompt_cached(sid, p)
        ohit, oslots, opair = ox.alloc_prompt_cached(sid, p)
        assert hit == ohit and list(slots) == oslots and pair == opair
        assert hit == {0: 331, 1: 213, 2: len(sc.tokens[1]), 3: 0}[k]
        if pair is not None:
            pa.pa_copy_blocks(sc.pool, torch.tensor([pair], dtype=torch.int32, device="cuda"))
            C.copy_blocks(sc.ok, [pair], sc.oks)
            C.copy_blocks(sc.ov, [pair], sc.ovs)
        sc._write(oslots, len(oslots))       # the suffix's own K/V
        sc.seqs.append(sid)
        seqs.append(sid)
        suffix.append(len(p) - hit)
    sc.check_pool_bits()
    qsl = np.concatenate([[0], np.cumsum(suffix)]).astype(np.int32)
    q_dev, q64 = sc.random_q(int(qsl[-1]), kv)
    scale = 1 / math.sqrt(D)
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, kv, tables, lens, bs, scale)
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    out = torch.full(q_dev.shape, float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_prefill_chunk(out, q_dev, sc.pool, t_dev, ln_dev, torch.from_numpy(qsl).cuda(),
                        int(max(suffix)), scale)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy().astype(np.float64), ref, TOL[kv], f"suffix prefill {kv} bs={bs}")
    # the cached rows are the rows written for the entry that provides them:
    # prompt 1's first 213 rows are sequence 0's (freed, kept by the index)
    g1 = C.gather(sc.ok, sc.ora.block_table(11), 213, bs)
    g_src = C.gather(sc.ok, ox.entries[0][1], 213, bs)
    assert np.array_equal(g1, g_src)
