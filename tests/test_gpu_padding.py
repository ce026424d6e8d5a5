"""Block-table padding is never read as a block id: with the entries past
each sequence's ceil(L / block_size) blocks filled with garbage (huge,
negative, out-of-pool ids) instead of -1, every GPU call returns the same
bits as with -1 padding."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_166_amd as pa
from tests.gpu_util import Scenario

pytestmark = pytest.mark.gpu


def _garbage(t, ln, bs, seed):
    """A copy of host tables t with every padding entry replaced by garbage."""
    rng = np.random.default_rng(seed)
    g = t.copy()
    for i, L in enumerate(ln):
        n = -(-int(L) // bs)
        k = g.shape[1] - n
        if k > 0:
            g[i, n:] = rng.choice(np.array([2 ** 31 - 1, -2 ** 31, 1 << 28, -7, 123456789],
                                           dtype=np.int64), k).astype(np.int32)
    return g


def _bits(x):
    return x.view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("kv", ["f16", "fp8"])
def test_decode_ignores_table_padding(kv):
    bs, H, D = 16, 2, 128
    lens = [0, 1, 15, 16, 17, 100, 700]
    N = sum(-(-L // bs) for L in lens) + 6
    sc = Scenario(N, H, bs, D, kv, seed=81)
    for i, L in enumerate(lens):
        sc.prompt(i, L)
    seqs = list(range(len(lens)))
    q, _ = sc.random_q(len(seqs), "bf16" if kv == "fp8" else kv)
    t, ln = sc.tables(seqs, max_blocks=64)            # every row padded
    ln_d = torch.from_numpy(ln).cuda()
    for pb in (0, 1, 3):
        outs = []
        for tab in (t, _garbage(t, ln, bs, pb)):
            out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
            pa.pa_decode(out, q, sc.pool, torch.from_numpy(tab).cuda(), ln_d, 0.1, pb,
                         pa.decode_workspace(sc.pool, len(seqs), tab.shape[1], pb))
            outs.append(out)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(outs[0]), _bits(outs[1])), f"{kv} pb={pb}"


def test_prefill_ignores_table_padding():
    bs, H, D = 16, 2, 128
    ctx, chunk = [0, 33, 100, 5], [7, 40, 129, 1]
    N = sum(-(-(c + s) // bs) for c, s in zip(ctx, chunk)) + 4
    sc = Scenario(N, H, bs, D, "bf16", seed=82)
    for i, (c, s) in enumerate(zip(ctx, chunk)):
        sc.prompt(i, c)
        sc.append(i, s)
    seqs = list(range(len(ctx)))
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(chunk)]), dtype=torch.int32, device="cuda")
    q, _ = sc.random_q(int(sum(chunk)), "bf16")
    t, ln = sc.tables(seqs, max_blocks=40)
    ln_d = torch.from_numpy(ln).cuda()
    outs = []
    for tab in (t, _garbage(t, ln, bs, 5)):
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        pa.pa_prefill_chunk(out, q, sc.pool, torch.from_numpy(tab).cuda(), ln_d, qsl, 129,
                            1 / math.sqrt(D))
        outs.append(out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(outs[0]), _bits(outs[1]))


def test_shared_prefix_and_append_ignore_table_padding():
    bs, H, D = 16, 2, 128
    own = [0, 3, 40, 17]
    N = 4 + sum(-(-n // bs) for n in own) + len(own) + 4
    sc = Scenario(N, H, bs, D, "f16", seed=83)
    sc.prompt(0, 4 * bs)
    for i in range(1, len(own)):
        sc.fork(0, i)
    for i, n in enumerate(own):
        if n:
            sc.append(i, n)
    seqs = list(range(len(own)))
    q, _ = sc.random_q(len(seqs), "f16")
    t, ln = sc.tables(seqs, max_blocks=32)
    ln_d = torch.from_numpy(ln).cuda()
    outs = []
    for tab in (t, _garbage(t, ln, bs, 9)):
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        pa.pa_decode_shared_prefix(out, q, sc.pool, torch.from_numpy(tab).cuda(), ln_d, 4, 0.1)
        outs.append(out)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(outs[0]), _bits(outs[1]))
    # pa_decode_append: the step's row stored at a slot of each sequence's
    # last block (position L - 1 after one more token), same outputs and pool
    # bits either way
    k_new = torch.randn(q.shape, device="cuda").to(torch.float16)
    v_new = torch.randn(q.shape, device="cuda").to(torch.float16)
    res = []
    for tab in (t, _garbage(t, ln, bs, 11)):
        sc2 = Scenario(N, H, bs, D, "f16", seed=83)
        sc2.prompt(0, 4 * bs)
        for i in range(1, len(own)):
            sc2.fork(0, i)
        for i, n in enumerate(own):
            if n:
                sc2.append(i, n)
        slots = []
        for i in seqs:
            s, cow = sc2.alloc.append_tokens(i, 1)
            assert cow is None                 # every last block is unshared or full
            slots.append(s[0])
        t2, ln2 = sc2.alloc.pack(seqs, 32)
        g2 = t2 if tab is t else _garbage(t2, ln2, bs, 11)
        out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        pa.pa_decode_append(out, q, sc2.pool, k_new, v_new,
                            torch.tensor(slots, dtype=torch.int64, device="cuda"),
                            torch.from_numpy(g2).cuda(), torch.from_numpy(ln2).cuda(), 0.1)
        torch.cuda.synchronize()
        res.append((_bits(out), sc2.pool.k_cache.view(torch.int16).cpu().numpy(),
                    sc2.pool.v_cache.view(torch.int16).cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)
