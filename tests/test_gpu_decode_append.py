"""pa_decode_append (the step's new K/V row stored and attended in one
launch) against pa_reshape_and_cache followed by pa_decode: bit for bit in
the outputs and in the whole pool, over dtypes, head sizes, block sizes
(new rows at the first, a middle and the last position of a block, a
one-token sequence, a sequence without a new row), partition sizes and the
stream flag; and against the oracle."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_166_amd as pa
from oracle import cache as C
from tests.gpu_util import (TOL, Scenario, assert_close, bits_to_device, device_bits, to_bits,
                            values_f64)
from tests.test_gpu_decode import _oracle

pytestmark = pytest.mark.gpu


def _clone(pool):
    return pa.PagedPool(pool.k_cache.clone(), pool.v_cache.clone(), kv_dtype=pool.kv_dtype,
                        stream_kv=pool.stream_kv)


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [4, 8, 16, 32, 64])
def test_append_equals_write_then_decode(kv, D, bs):
    H = 3
    lens = sorted({1, 2, bs, bs + 1, 2 * bs, 3 * bs - 1, 150, 600})   # lengths after the append
    N = sum(-(-L // bs) for L in lens) + 5
    sc = Scenario(N, H, bs, D, kv, seed=80 + D + bs)
    for i, L in enumerate(lens):
        sc.prompt(i, L - 1)
    seqs = list(range(len(lens)))
    slots = []
    for i in seqs:
        s_lib, cow = sc.alloc.append_tokens(i, 1)
        s_ora, _ = sc.ora.append_tokens(i, 1)
        assert list(s_lib) == s_ora and cow is None
        slots += s_ora
    slots[3] = -1                            # no new row for this one: its last row stays unwritten
    rng = np.random.default_rng(D + bs)
    kb = to_bits(rng.standard_normal((len(seqs), H, D), dtype=np.float32), kv)
    vb = to_bits(rng.standard_normal((len(seqs), H, D), dtype=np.float32), kv)
    kn, vn = bits_to_device(kb, kv, "cuda"), bits_to_device(vb, kv, "cuda")
    sl = torch.tensor(slots, dtype=torch.int64, device="cuda")
    q_dev, q64 = sc.random_q(len(seqs), kv)
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    scale = 1 / math.sqrt(D)
    base_k, base_v = sc.pool.k_cache.clone(), sc.pool.v_cache.clone()
    # the oracle: the same rows written, then attention
    C.write_rows(sc.ok, kb, slots, bs)
    C.write_rows(sc.ov, vb, slots, bs)
    ref = _oracle(sc, seqs, q64, scale)
    for stream in (False, True):
        for pb in (0, 1, 3):
            sc.pool.k_cache.copy_(base_k)
            sc.pool.v_cache.copy_(base_v)
            sc.pool.stream_kv = stream
            two = _clone(sc.pool)
            pa.pa_reshape_and_cache(two, kn, vn, sl)
            out2 = torch.empty((len(seqs), H, D), dtype=torch.float32, device="cuda")
            pa.pa_decode(out2, q_dev, two, t_dev, ln_dev, scale, pb,
                         pa.decode_workspace(two, len(seqs), t_dev.shape[1], pb))
            out1 = torch.full((len(seqs), H, D), float("nan"), dtype=torch.float32, device="cuda")
            pa.pa_decode_append(out1, q_dev, sc.pool, kn, vn, sl, t_dev, ln_dev, scale, pb,
                                pa.decode_workspace(sc.pool, len(seqs), t_dev.shape[1], pb))
            torch.cuda.synchronize()
            what = f"{kv} D={D} bs={bs} pb={pb} stream={stream}"
            assert np.array_equal(out1.cpu().numpy().view(np.uint32),
                                  out2.cpu().numpy().view(np.uint32)), what
            assert np.array_equal(device_bits(sc.pool.k_cache), device_bits(two.k_cache)), what
            assert np.array_equal(device_bits(sc.pool.v_cache), device_bits(two.v_cache)), what
            got = out1.cpu().numpy().astype(np.float64)
            keep = [i for i in seqs if i != 3]     # seq 3 reads its unwritten (sentinel) last row
            assert_close(got[keep], ref[keep], TOL[kv], what)
    sc.check_pool_bits()                     # the oracle's pool, rows written once


@pytest.mark.parametrize("auto", [False, True])
@pytest.mark.parametrize("qdt", ["bf16", "f16"])
@pytest.mark.parametrize("D,bs", [(128, 32), (128, 16), (64, 4), (128, 64), (64, 64)])
def test_fp8_append_equals_write_then_decode(auto, qdt, D, bs):
    """fp8 pools: the new rows (of q's type) quantised by the decode launch --
    with the blocks' scales kept up (PA_POOL_FP8_AUTO_SCALE: new rows whose
    amplitude grows the block's amax requantise its earlier rows, rows that
    start a block set a fresh scale) or with the caller's scales -- against
    pa_reshape_and_cache of the same rows followed by pa_decode: outputs,
    codes and scales bit for bit; then against the oracle at the fp8
    tolerance."""
    H = 3
    lens = sorted({1, 2, bs, bs + 1, 2 * bs, 3 * bs - 1, 150, 600})   # lengths after the append
    N = sum(-(-L // bs) for L in lens) + 5
    sc = Scenario(N, H, bs, D, "fp8", seed=90 + D + bs, in_dtype=qdt,
                  scale_range=(0.011, 0.03), fp8_auto_scale=auto)
    rng = np.random.default_rng(D + bs + auto)
    for i, L in enumerate(lens):
        sc.prompt(i, L - 1, amp=rng.uniform(0.2, 2.0, (max(L - 1, 1), H, 1))[:L - 1])
    seqs = list(range(len(lens)))
    slots = []
    for i in seqs:
        s_lib, cow = sc.alloc.append_tokens(i, 1)
        s_ora, _ = sc.ora.append_tokens(i, 1)
        assert list(s_lib) == s_ora and cow is None
        slots += s_ora
    slots[3] = -1                            # no new row for this one
    amp = rng.choice([0.05, 1.0, 30.0], size=(len(seqs), H, 1)).astype(np.float32)
    kb = to_bits(rng.standard_normal((len(seqs), H, D), dtype=np.float32) * amp, qdt)
    vb = to_bits(rng.standard_normal((len(seqs), H, D), dtype=np.float32) * amp, qdt)
    kn, vn = bits_to_device(kb, qdt, "cuda"), bits_to_device(vb, qdt, "cuda")
    sl = torch.tensor(slots, dtype=torch.int64, device="cuda")
    q_dev, q64 = sc.random_q(len(seqs), qdt)
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    scale = 1 / math.sqrt(D)
    p = sc.pool
    base = [t.clone() for t in (p.k_cache, p.v_cache, p.k_scale, p.v_scale)]
    # the oracle: the same rows written (with or without scale upkeep), then attention
    w = C.write_rows_fp8_upkeep if auto else C.write_rows_fp8
    kf = values_f64(kb, qdt).astype(np.float32)
    vf = values_f64(vb, qdt).astype(np.float32)
    w(sc.ok, kf, slots, sc.oks, bs)
    w(sc.ov, vf, slots, sc.ovs, bs)
    ref = _oracle(sc, seqs, q64, scale)
    for pb in (0, 1, 3):
        for t, b in zip((p.k_cache, p.v_cache, p.k_scale, p.v_scale), base):
            t.copy_(b)
        two = pa.PagedPool(p.k_cache.clone(), p.v_cache.clone(), p.k_scale.clone(),
                           p.v_scale.clone(), kv_dtype=p.kv_dtype, fp8_auto_scale=auto)
        pa.pa_reshape_and_cache(two, kn, vn, sl)
        out2 = torch.empty((len(seqs), H, D), dtype=torch.float32, device="cuda")
        pa.pa_decode(out2, q_dev, two, t_dev, ln_dev, scale, pb,
                     pa.decode_workspace(two, len(seqs), t_dev.shape[1], pb))
        out1 = torch.full((len(seqs), H, D), float("nan"), dtype=torch.float32, device="cuda")
        pa.pa_decode_append(out1, q_dev, p, kn, vn, sl, t_dev, ln_dev, scale, pb,
                            pa.decode_workspace(p, len(seqs), t_dev.shape[1], pb))
        torch.cuda.synchronize()
        what = f"fp8 auto={auto} q={qdt} D={D} bs={bs} pb={pb}"
        assert np.array_equal(out1.cpu().numpy().view(np.uint32),
                              out2.cpu().numpy().view(np.uint32)), what
        for a_, b_ in ((p.k_cache, two.k_cache), (p.v_cache, two.v_cache),
                       (p.k_scale, two.k_scale), (p.v_scale, two.v_scale)):
            assert np.array_equal(device_bits(a_), device_bits(b_)), what
        got = out1.cpu().numpy().astype(np.float64)
        keep = [i for i in seqs if i != 3]     # seq 3 reads its unwritten (sentinel) last row
        assert_close(got[keep], ref[keep], TOL["fp8"], what)
    sc.check_pool_bits()                     # codes and scales against the oracle's


def _append_step(sc, seqs, stream):
    """One decode step as the bench runs it: batch append in the allocators,
    copies for shared last blocks, then pa_decode_append with the new rows."""
    import workloads as W  # noqa: F401
    slots_lib, cow_lib, _ = sc.alloc.append_tokens_batch(seqs, 1)
    want = sc.ora.append_tokens_batch(seqs, 1)
    assert [list(r) for r in slots_lib] == [w[0] for w in want]
    pairs = [w[1] for w in want if w[1] is not None]
    if pairs:
        pa.pa_copy_blocks(sc.pool, torch.tensor(pairs, dtype=torch.int32, device="cuda"))
        C.copy_blocks(sc.ok, pairs)
        C.copy_blocks(sc.ov, pairs)
    slots = [w[0][0] for w in want]
    H, D, kv = sc.H, sc.D, sc.kv
    kb = to_bits(sc.rng.standard_normal((len(seqs), H, D), dtype=np.float32), kv)
    vb = to_bits(sc.rng.standard_normal((len(seqs), H, D), dtype=np.float32), kv)
    C.write_rows(sc.ok, kb, slots, sc.bs)
    C.write_rows(sc.ov, vb, slots, sc.bs)
    q_dev, q64 = sc.random_q(len(seqs), kv)
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    sc.pool.stream_kv = stream
    out = torch.full((len(seqs), H, D), float("nan"), dtype=torch.float32, device="cuda")
    pa.pa_decode_append(out, q_dev, sc.pool, bits_to_device(kb, kv, "cuda"),
                        bits_to_device(vb, kv, "cuda"),
                        torch.tensor(slots, dtype=torch.int64, device="cuda"), t_dev, ln_dev,
                        1 / math.sqrt(D), 0, pa.decode_workspace(sc.pool, len(seqs), t_dev.shape[1]))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), q64, len(pairs)


def test_llama13b_step_as_benchmarked():
    """The LLaMA-13B decode batch (32 sequences of 128..2048 tokens after the
    step, 40 heads x 128, fp16, block 16, shuffled 4096-block pool), one step
    through pa_decode_append with the stream flag: the whole pool bit for bit
    and all 1280 outputs against the oracle."""
    import workloads as W
    cfg = W.CONFIGS["llama13b_decode"]
    lens = W.uniform_ints(cfg["seed"], cfg["batch"], cfg["len_lo"], cfg["len_hi"])
    sc = Scenario(cfg["num_blocks"], cfg["num_heads"], cfg["block_size"], cfg["head_dim"], "f16",
                  seed=cfg["seed"])
    for i, L in enumerate(lens):
        sc.prompt(i, int(L) - 1)
    seqs = list(range(cfg["batch"]))
    got, q64, ncow = _append_step(sc, seqs, stream=True)
    assert ncow == 0
    sc.check_pool_bits()
    ref = _oracle(sc, seqs, q64, 1 / math.sqrt(cfg["head_dim"]))
    assert_close(got, ref, TOL["f16"], "llama13b append step")


def test_prefix_cow_step_as_benchmarked():
    """64 sequences sharing a 1024-token prefix plus 1..256 own tokens (bf16,
    block 16), one step through pa_decode_append; then a fork in the middle of
    a block whose next step copies the shared block before the new row is
    stored by the decode launch."""
    import workloads as W
    cfg = W.CONFIGS["prefix_cow"]
    B = cfg["batch"]
    sc = Scenario(cfg["num_blocks"], cfg["num_heads"], cfg["block_size"], cfg["head_dim"], "bf16",
                  seed=cfg["seed"])
    sc.prompt(0, cfg["prefix"])
    for i in range(1, B):
        sc.fork(0, i)
    suffix = W.uniform_ints(cfg["seed"], B, cfg["suffix_lo"], cfg["suffix_hi"])
    for i in range(B):
        sc.append(i, int(suffix[i]))
    seqs = list(range(B))
    scale = 1 / math.sqrt(cfg["head_dim"])
    got, q64, _ = _append_step(sc, seqs, stream=False)
    sc.check_pool_bits()
    assert_close(got, _oracle(sc, seqs, q64, scale), TOL["bf16"], "prefix append step")
    p = next(i for i in range(B) if sc.ora.seq_len(i) % cfg["block_size"] != 0)
    sc.fork(p, B)
    got2, q2, ncow = _append_step(sc, [p, B], stream=False)
    assert ncow == 1                         # the child's write copies the shared block first
    sc.check_pool_bits()
    assert_close(got2, _oracle(sc, [p, B], q2, scale), TOL["bf16"], "after CoW")
