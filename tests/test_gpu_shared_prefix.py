"""pa_decode_shared_prefix (the shared prefix attended once for the whole
batch on MFMA, each sequence's own blocks by the decode kernel, then one
merge) against the oracle and against pa_decode: block sizes, head sizes,
both 16-bit types, prefixes of one block, of a length that is no multiple of
the 32-key tile, and long enough to take wider chunks; batches of one and of
more than one 128-row tile; sequences with no tokens after the prefix;
several suffix partition sizes."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_166_amd as pa
from tests.gpu_util import TOL, Scenario, assert_close, half_ulp
from tests.test_gpu_decode import _oracle

pytestmark = pytest.mark.gpu


def _batch(kv, D, bs, H, shared_blocks, own, seed, **kw):
    """Sequence 0 holds the prefix; the others fork it; then own tokens."""
    N = shared_blocks + sum(-(-n // bs) for n in own) + len(own) + 4
    sc = Scenario(N, H, bs, D, kv, seed=seed, **kw)
    sc.prompt(0, shared_blocks * bs)
    for i in range(1, len(own)):
        sc.fork(0, i)
    for i, n in enumerate(own):
        if n:
            assert sc.append(i, n) is None          # the prefix ends on a block boundary
    return sc


def _run(sc, seqs, q_dev, shared_blocks, scale, pb=0, out_dtype=torch.float32):
    t_dev, ln_dev, t, ln = sc.device_tables(seqs)
    assert pa.shared_prefix_blocks(t, ln, sc.bs) >= shared_blocks
    out = torch.full(q_dev.shape, float("nan"), dtype=out_dtype, device="cuda")
    pa.pa_decode_shared_prefix(out, q_dev, sc.pool, t_dev, ln_dev, shared_blocks, scale, pb)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kv", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [4, 16, 32, 64])
def test_sweep(kv, D, bs):
    H = 3
    for shared_blocks, own in [(1, [0, 1, 5, 40]),
                               (max(1, 100 // bs), [3, 0, 77, 200, 1]),
                               (max(1, 600 // bs), [int(x) for x in np.arange(131) % 37])]:
        sc = _batch(kv, D, bs, H, shared_blocks, own, seed=bs + D + shared_blocks)
        seqs = list(range(len(own)))
        q_dev, q64 = sc.random_q(len(seqs), kv)
        scale = 1 / math.sqrt(D)
        ref = _oracle(sc, seqs, q64, scale)
        for pb in (0, 1, 3):
            got = _run(sc, seqs, q_dev, shared_blocks, scale, pb)
            assert_close(got, ref, TOL[kv], f"{kv} D={D} bs={bs} prefix={shared_blocks} pb={pb}")
        got = _run(sc, seqs, q_dev, shared_blocks, scale, 0, out_dtype=pa.TORCH_DTYPE[kv])
        assert np.all(np.abs(got - ref) <= TOL[kv] + half_ulp(kv, ref)), "low-precision output"


def test_long_prefix_takes_wider_chunks():
    """A 20480-token prefix (more than 64 chunks of 256 keys, so the chunks
    widen to 320 keys)."""
    sc = _batch("bf16", 128, 64, 2, 320, [0, 9, 130, 64], seed=9)
    seqs = [0, 1, 2, 3]
    q_dev, q64 = sc.random_q(4, "bf16")
    ref = _oracle(sc, seqs, q64, 0.1)
    assert_close(_run(sc, seqs, q_dev, 320, 0.1), ref, TOL["bf16"], "long prefix")


def test_prefix_cow_workload():
    """The shared-prefix workload's decode step (64 sequences, 1024-token
    prefix in 64 blocks of 16, 1..256 own tokens plus the step's, 40 heads x
    128, bf16): every output against the oracle and against pa_decode."""
    import workloads as W
    cfg = W.CONFIGS["prefix_cow"]
    own = [int(s) + 1 for s in W.uniform_ints(cfg["seed"], cfg["batch"], cfg["suffix_lo"],
                                              cfg["suffix_hi"])]
    sc = _batch("bf16", cfg["head_dim"], cfg["block_size"], cfg["num_heads"],
                cfg["prefix"] // cfg["block_size"], own, seed=cfg["seed"])
    seqs = list(range(cfg["batch"]))
    q_dev, q64 = sc.random_q(len(seqs), "bf16")
    scale = 1 / math.sqrt(cfg["head_dim"])
    ref = _oracle(sc, seqs, q64, scale)
    got = _run(sc, seqs, q_dev, cfg["prefix"] // cfg["block_size"], scale)
    err = assert_close(got, ref, TOL["bf16"], "shared-prefix decode")
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    plain = torch.empty(q_dev.shape, dtype=torch.float32, device="cuda")
    pa.pa_decode(plain, q_dev, sc.pool, t_dev, ln_dev, scale, 0,
                 pa.decode_workspace(sc.pool, len(seqs), t_dev.shape[1]))
    torch.cuda.synchronize()
    assert_close(got, plain.cpu().numpy().astype(np.float64), TOL["bf16"], "against pa_decode")
    print(f"shared-prefix decode: max abs err {err:.2e}")


def test_refusals():
    sc = Scenario(8, 2, 16, 128, "fp8", seed=3)
    sc.prompt(0, 32)
    t_dev, ln_dev, _, _ = sc.device_tables([0])
    q = torch.zeros((1, 2, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((1, 2, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(NotImplementedError):                   # fp8 pool, f32 queries
        pa.pa_decode_shared_prefix(out, q.float(), sc.pool, t_dev, ln_dev, 1, 0.1, 0, ws)
    sc3 = Scenario(8, 2, 16, 128, "f32", seed=3)
    sc3.prompt(0, 32)
    t3, l3, _, _ = sc3.device_tables([0])
    with pytest.raises(NotImplementedError):                   # f32 pool
        pa.pa_decode_shared_prefix(out, q.float(), sc3.pool, t3, l3, 1, 0.1, 0, ws)
    sc2 = Scenario(8, 2, 16, 128, "bf16", seed=3)
    sc2.prompt(0, 32)
    t2, l2, _, _ = sc2.device_tables([0])
    with pytest.raises(ValueError):
        pa.pa_decode_shared_prefix(out, q, sc2.pool, t2, l2, 0, 0.1, 0, ws)   # no shared block
    with pytest.raises(ValueError):
        pa.pa_decode_shared_prefix(out, q, sc2.pool, t2, l2, 1, 0.1, 0, ws[:16])  # workspace


@pytest.mark.parametrize("qdt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 64])
def test_fp8_pool(qdt, D, bs):
    """fp8 E4M3 pools with f16 or bf16 queries: the prefix pass over the
    codes and their scales, against the oracle (tolerance 2e-2) and against
    pa_decode of the same batch."""
    H = 3
    for shared_blocks, own in [(1, [0, 1, 5, 40]), (max(1, 600 // bs), [3, 0, 77, 200, 1])]:
        sc = _batch("fp8", D, bs, H, shared_blocks, own, seed=bs + D + shared_blocks,
                    in_dtype=qdt, scale_range=(0.011, 0.03))
        seqs = list(range(len(own)))
        q_dev, q64 = sc.random_q(len(seqs), qdt)
        scale = 1 / math.sqrt(D)
        ref = _oracle(sc, seqs, q64, scale)
        got = _run(sc, seqs, q_dev, shared_blocks, scale)
        err = assert_close(got, ref, TOL["fp8"], f"fp8 q={qdt} D={D} bs={bs} prefix={shared_blocks}")
        assert err / np.max(np.abs(ref)) < 5e-3
        t_dev, ln_dev, _, _ = sc.device_tables(seqs)
        plain = torch.empty(q_dev.shape, dtype=torch.float32, device="cuda")
        pa.pa_decode(plain, q_dev, sc.pool, t_dev, ln_dev, scale, 0,
                     pa.decode_workspace(sc.pool, len(seqs), t_dev.shape[1]))
        torch.cuda.synchronize()
        assert np.max(np.abs(got - plain.cpu().numpy())) < 1e-3


@pytest.mark.parametrize("kv", ["bf16", "f16"])
@pytest.mark.parametrize("bs", [4, 16, 64])
def test_append_equals_write_then_shared_prefix(kv, bs):
    """pa_decode_shared_prefix_append (the step's new rows stored and attended
    in the launch) against pa_reshape_and_cache followed by
    pa_decode_shared_prefix: bit for bit in the outputs and in the whole
    pool, with the merge fused into the decode launch (automatic partitions)
    and in its own launch (one-block partitions); and against the oracle.
    One sequence has no tokens past the prefix before the step, one gets no
    new row."""
    from oracle import cache as C
    from tests.gpu_util import bits_to_device, device_bits, to_bits
    D, H = 128, 3
    shared_blocks = max(1, 100 // bs)
    own = [3, 0, 77, 200, 1, bs - 1]
    sc = _batch(kv, D, bs, H, shared_blocks, own, seed=300 + bs)
    seqs = list(range(len(own)))
    slots = []
    for i in seqs:
        s_lib, cow = sc.alloc.append_tokens(i, 1)
        s_ora, _ = sc.ora.append_tokens(i, 1)
        assert list(s_lib) == s_ora and cow is None
        slots += s_ora
    slots[4] = -1                            # no new row for this one
    rng = np.random.default_rng(bs)
    kb = to_bits(rng.standard_normal((len(seqs), H, D), dtype=np.float32), kv)
    vb = to_bits(rng.standard_normal((len(seqs), H, D), dtype=np.float32), kv)
    kn, vn = bits_to_device(kb, kv, "cuda"), bits_to_device(vb, kv, "cuda")
    sl = torch.tensor(slots, dtype=torch.int64, device="cuda")
    q_dev, q64 = sc.random_q(len(seqs), kv)
    t_dev, ln_dev, t, ln = sc.device_tables(seqs)
    assert pa.shared_prefix_blocks(t, ln, bs) >= shared_blocks
    scale = 1 / math.sqrt(D)
    base_k, base_v = sc.pool.k_cache.clone(), sc.pool.v_cache.clone()
    C.write_rows(sc.ok, kb, slots, bs)
    C.write_rows(sc.ov, vb, slots, bs)
    ref = _oracle(sc, seqs, q64, scale)
    for pb in (0, 1):
        outs, pools = [], []
        for fused in (False, True):
            sc.pool.k_cache.copy_(base_k)
            sc.pool.v_cache.copy_(base_v)
            out = torch.full(q_dev.shape, float("nan"), dtype=torch.float32, device="cuda")
            if fused:
                pa.pa_decode_shared_prefix_append(out, q_dev, sc.pool, kn, vn, sl, t_dev, ln_dev,
                                                  shared_blocks, scale, pb)
            else:
                pa.pa_reshape_and_cache(sc.pool, kn, vn, sl)
                pa.pa_decode_shared_prefix(out, q_dev, sc.pool, t_dev, ln_dev, shared_blocks,
                                           scale, pb)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
            pools.append((device_bits(sc.pool.k_cache), device_bits(sc.pool.v_cache)))
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), f"pb={pb}"
        assert np.array_equal(pools[0][0], pools[1][0]) and np.array_equal(pools[0][1], pools[1][1])
        assert np.array_equal(pools[1][0], sc.ok) and np.array_equal(pools[1][1], sc.ov)
        assert_close(outs[1].astype(np.float64), ref, TOL[kv], f"{kv} bs={bs} pb={pb}")
