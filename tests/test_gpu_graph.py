"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph): a
decode step (cache write, pa_decode with its split-K merge, and
pa_decode_append) and a prefill chunk, captured once and replayed several
times with eager work and synchronisations in between; every replay gives
the eager result bit for bit (no call records a memset or a host-side
dependency into the graph)."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_166_amd as pa
from tests.gpu_util import Scenario

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32).cpu().numpy().copy()


def test_decode_step_replays():
    bs, H, D = 16, 4, 128
    lens = [1, 15, 300, 700, 33]
    N = sum(-(-(L + 1) // bs) for L in lens) + 8
    sc = Scenario(N, H, bs, D, "f16", seed=91)
    for i, L in enumerate(lens):
        sc.prompt(i, L)
    seqs = list(range(len(lens)))
    # the step: one new token per sequence
    slots = torch.tensor([sc.alloc.append_tokens(i, 1)[0][0] for i in seqs], dtype=torch.int64,
                         device="cuda")
    t, ln = sc.alloc.pack(seqs, 64)
    td, ld = torch.from_numpy(t).cuda(), torch.from_numpy(ln).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    q = torch.randn((len(seqs), H, D), generator=g, device="cuda").to(torch.float16)
    k_new = torch.randn((len(seqs), H, D), generator=g, device="cuda").to(torch.float16)
    v_new = torch.randn((len(seqs), H, D), generator=g, device="cuda").to(torch.float16)
    out1 = torch.empty((len(seqs), H, D), dtype=torch.float32, device="cuda")
    out2 = torch.empty_like(out1)
    ws1 = pa.decode_workspace(sc.pool, len(seqs), 64, 3)
    ws2 = pa.decode_workspace(sc.pool, len(seqs), 64, 0)
    k0, v0 = sc.pool.k_cache.clone(), sc.pool.v_cache.clone()

    def step():
        pa.pa_reshape_and_cache(sc.pool, k_new, v_new, slots)
        pa.pa_decode(out1, q, sc.pool, td, ld, 0.1, 3, ws1)
        pa.pa_decode_append(out2, q, sc.pool, k_new, v_new, slots, td, ld, 0.1, 0, ws2)

    step()                                    # eager reference
    torch.cuda.synchronize()
    ref = (_bits(out1), _bits(out2), sc.pool.k_cache.view(torch.int16).cpu().numpy().copy())
    sc.pool.k_cache.copy_(k0)
    sc.pool.v_cache.copy_(v0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()                                # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.synchronize()
    for r in range(4):
        out1.fill_(float("nan"))
        out2.fill_(float("nan"))
        sc.pool.k_cache.copy_(k0)             # eager work between the replays
        sc.pool.v_cache.copy_(v0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out1), ref[0]), f"replay {r}: pa_decode"
        assert np.array_equal(_bits(out2), ref[1]), f"replay {r}: pa_decode_append"
        assert np.array_equal(sc.pool.k_cache.view(torch.int16).cpu().numpy(), ref[2]), f"replay {r}"


def test_prefill_chunk_replays():
    bs, H, D = 32, 2, 128
    ctx, chunk = [0, 900, 37], [130, 300, 1]
    N = sum(-(-(c + s) // bs) for c, s in zip(ctx, chunk)) + 4
    sc = Scenario(N, H, bs, D, "bf16", seed=92)
    for i, (c, s) in enumerate(zip(ctx, chunk)):
        sc.prompt(i, c)
        sc.append(i, s)
    seqs = list(range(len(ctx)))
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(chunk)]), dtype=torch.int32, device="cuda")
    q, _ = sc.random_q(int(sum(chunk)), "bf16")
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")

    def step():
        pa.pa_prefill_chunk(out, q, sc.pool, t_dev, ln_dev, qsl, 300, 1 / math.sqrt(D))

    step()
    torch.cuda.synchronize()
    ref = _bits(out)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), ref), f"replay {r}"
