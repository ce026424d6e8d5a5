"""GPU parity of pa_prefill_chunk against the oracle: causal attention of a
query chunk over its paged context (bottom-right aligned mask), bf16 / fp16,
float32 accumulation, tolerance 2e-3."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_166_amd as pa
import workloads as W
from oracle import attention as A
from tests.gpu_util import TOL, Scenario, assert_close, half_ulp

pytestmark = pytest.mark.gpu


def _setup(sc, ctx, chunk, qdt):
    for i, (c, s) in enumerate(zip(ctx, chunk)):
        sc.prompt(i, c)
        sc.append(i, s)                       # the chunk's own K/V
    seqs = list(range(len(ctx)))
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev, q64 = sc.random_q(int(qsl[-1]), qdt)
    return seqs, qsl, q_dev, q64


def _run(sc, seqs, qsl, q_dev, scale, out_dtype=torch.float32):
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    out = torch.full(q_dev.shape, float("nan"), dtype=out_dtype, device="cuda")
    mq = int(np.max(np.diff(qsl))) if len(qsl) > 1 else 0
    pa.pa_prefill_chunk(out, q_dev, sc.pool, t_dev, ln_dev, torch.from_numpy(qsl).cuda(), mq, scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("kv", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [4, 16, 32, 64])
def test_prefill_sweep(kv, D, bs):
    """Context 0 / short / ragged, chunks of 1 .. 200 rows (partial query
    tiles), a shuffled NaN-filled pool."""
    ctx = [0, 5, 37, 130, 0]
    chunk = [17, 1, 128, 200, 129]
    N = sum(-(-(c + s) // bs) for c, s in zip(ctx, chunk)) + 5
    sc = Scenario(N, 2, bs, D, kv, seed=41 + bs + D)
    seqs, qsl, q_dev, q64 = _setup(sc, ctx, chunk, kv)
    scale = 1 / math.sqrt(D)
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, kv, tables, lens, bs, scale)
    got = _run(sc, seqs, qsl, q_dev, scale)
    assert_close(got, ref, TOL[kv], f"prefill {kv} D={D} bs={bs}")
    got = _run(sc, seqs, qsl, q_dev, scale, out_dtype=pa.TORCH_DTYPE[kv])
    assert np.all(np.abs(got - ref) <= TOL[kv] + half_ulp(kv, ref)), "low-precision output"


@pytest.mark.parametrize("nseq", [16, 24])
def test_prefill_dispatch_orders(nseq):
    """Both work orders of the launch: 16 sequences x 3 query tiles (48
    classes: longest work first, each workgroup ranking the classes) and 24
    (72 classes: pairs in order), 5 heads (an uneven number of heads per XCD),
    ragged contexts and chunks from 1 to 300 rows, some classes without rows."""
    rng = np.random.default_rng(61 + nseq)
    ctx = [int(c) for c in rng.integers(0, 400, nseq)]
    chunk = [int(c) for c in rng.integers(1, 301, nseq)]
    chunk[0] = 300                      # three query tiles
    bs = 16
    N = sum(-(-(c + s) // bs) for c, s in zip(ctx, chunk)) + 8
    sc = Scenario(N, 5, bs, 64, "bf16", seed=63 + nseq)
    seqs, qsl, q_dev, q64 = _setup(sc, ctx, chunk, "bf16")
    scale = 1 / math.sqrt(64)
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, "bf16", tables, lens, bs, scale)
    got = _run(sc, seqs, qsl, q_dev, scale)
    assert_close(got, ref, TOL["bf16"], f"dispatch order, {nseq} sequences")


def test_prefill_whole_sequence_is_causal_attention():
    """No earlier context: the chunk is the whole sequence (top-left mask)."""
    sc = Scenario(12, 3, 32, 128, "bf16", seed=45)
    seqs, qsl, q_dev, q64 = _setup(sc, [0, 0], [300, 64], "bf16")
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, "bf16", tables, lens, 32, 0.125)
    got = _run(sc, seqs, qsl, q_dev, 0.125)
    assert_close(got, ref, TOL["bf16"], "whole sequence")


def test_chunked_prefill_workload():
    """8 sequences, a 512-token chunk after 0..3584 tokens of context, 32 heads
    x 128, bf16, block 32, shuffled 4096-block pool: pool bit for bit, then
    every output of the full-size launch against the oracle (all 32 heads:
    the dispatch deals (sequence, head) pairs to the 8 XCDs by pair % 8)."""
    cfg = W.CONFIGS["chunked_prefill"]
    ctx = [int(c) for c in W.uniform_ints(cfg["seed"], cfg["batch"], cfg["ctx_lo"], cfg["ctx_hi"])]
    chunk = [cfg["chunk"]] * cfg["batch"]
    sc = Scenario(cfg["num_blocks"], cfg["num_heads"], cfg["block_size"], cfg["head_dim"], "bf16",
                  seed=cfg["seed"])
    seqs, qsl, q_dev, q64 = _setup(sc, ctx, chunk, "bf16")
    sc.check_pool_bits()
    scale = 1 / math.sqrt(cfg["head_dim"])
    got = _run(sc, seqs, qsl, q_dev, scale)
    assert np.all(np.isfinite(got))
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, "bf16", tables, lens, cfg["block_size"], scale)
    err = assert_close(got, ref, TOL["bf16"], "chunked prefill")
    rel = err / np.max(np.abs(ref))
    print(f"chunked prefill: ctx={ctx} max abs err {err:.2e}, rel {rel:.2e}")
    assert rel < 5e-3, f"relative error {rel:.2e}"


def test_prefill_empty_chunks_and_no_op_calls():
    """Sequences with no query rows in the batch (first, middle and last),
    max_query_len above every chunk, and the calls that do nothing (no
    sequences, max_query_len 0), which leave out untouched."""
    ctx = [40, 7, 0, 300, 64, 33]
    chunk = [0, 33, 1, 0, 130, 0]
    bs = 16
    N = sum(-(-(c + s) // bs) for c, s in zip(ctx, chunk)) + 4
    sc = Scenario(N, 2, bs, 128, "f16", seed=47)
    for i, (c, s) in enumerate(zip(ctx, chunk)):
        sc.prompt(i, c)
        if s:
            sc.append(i, s)
    seqs = list(range(len(ctx)))
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q_dev, q64 = sc.random_q(int(qsl[-1]), "f16")
    scale = 1 / math.sqrt(128)
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, "f16", tables, lens, bs, scale)
    t_dev, ln_dev, _, _ = sc.device_tables(seqs)
    qsl_dev = torch.from_numpy(qsl).cuda()
    for mq in (130, 300):
        out = torch.full(q_dev.shape, float("nan"), dtype=torch.float32, device="cuda")
        pa.pa_prefill_chunk(out, q_dev, sc.pool, t_dev, ln_dev, qsl_dev, mq, scale)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().astype(np.float64), ref, TOL["f16"], f"empty chunks mq={mq}")
    out = torch.full(q_dev.shape, 7.0, dtype=torch.float32, device="cuda")
    pa.pa_prefill_chunk(out, q_dev, sc.pool, t_dev[:0], ln_dev[:0], qsl_dev[:1], 130, scale)
    pa.pa_prefill_chunk(out, q_dev, sc.pool, t_dev, ln_dev, qsl_dev, 0, scale)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


@pytest.mark.parametrize("qdt", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [4, 8, 16, 32, 64])
def test_prefill_fp8_pool(qdt, D, bs):
    """fp8 E4M3 pools (per-(block, head) scales) with bf16 or fp16 queries:
    contexts 0 .. 700, chunks of 1 .. 200 rows, against the oracle fed the
    same codes and scales (tolerance 2e-2; the codes are exact in 16 bits,
    only the scaled weights are rounded)."""
    ctx = [0, 5, 37, 700, 130]
    chunk = [17, 1, 128, 200, 129]
    N = sum(-(-(c + s) // bs) for c, s in zip(ctx, chunk)) + 5
    sc = Scenario(N, 2, bs, D, "fp8", seed=51 + bs + D, in_dtype=qdt, scale_range=(0.011, 0.03))
    seqs, qsl, q_dev, q64 = _setup(sc, ctx, chunk, qdt)
    scale = 1 / math.sqrt(D)
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, "fp8", tables, lens, bs, scale,
                          k_scale=sc.oks, v_scale=sc.ovs)
    got = _run(sc, seqs, qsl, q_dev, scale)
    err = assert_close(got, ref, TOL["fp8"], f"fp8 prefill q={qdt} D={D} bs={bs}")
    rel = err / np.max(np.abs(ref))
    assert rel < 5e-3, f"relative error {rel:.2e}"
    got = _run(sc, seqs, qsl, q_dev, scale, out_dtype=pa.TORCH_DTYPE[qdt])
    assert np.all(np.abs(got - ref) <= TOL["fp8"] + half_ulp(qdt, ref)), "low-precision output"


def test_prefill_fp8_chunked_workload_shape():
    """The chunked-prefill shape (512-row chunks, 32 heads x 128, block 32)
    over an fp8 pool with bf16 queries, contexts up to 2500: every output
    against the oracle fed the same codes and scales."""
    ctx = [2500, 0, 977, 31]
    chunk = [512, 512, 300, 512]
    bs, H, D = 32, 32, 128
    N = sum(-(-(c + s) // bs) for c, s in zip(ctx, chunk)) + 3
    sc = Scenario(N, H, bs, D, "fp8", seed=57, in_dtype="bf16", scale_range=(0.011, 0.03))
    seqs, qsl, q_dev, q64 = _setup(sc, ctx, chunk, "bf16")
    scale = 1 / math.sqrt(D)
    got = _run(sc, seqs, qsl, q_dev, scale)
    tables, lens = sc.oracle_tables(seqs)
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, "fp8", tables, lens, bs, scale,
                          k_scale=sc.oks, v_scale=sc.ovs)
    err = assert_close(got, ref, TOL["fp8"], "fp8 chunked prefill")
    rel = err / np.max(np.abs(ref))
    print(f"fp8 chunked prefill: max abs err {err:.2e}, rel {rel:.2e}")
    assert rel < 5e-3, f"relative error {rel:.2e}"


def test_prefill_bf16_value_range():
    """bf16 pools: the P V product runs on fp16 inputs, so V must stay within
    +-65504.  Just inside (+-65280, the largest bf16 below it) the output
    matches the oracle; just outside (2^16, which becomes inf) the outputs
    of that value's (head, dimension) turn inf or NaN for every row that
    sees the key, while rows far before it, the other dimensions and the
    other heads stay exact.  The same bound holds for the prefix pass of
    pa_decode_shared_prefix."""
    S, p = 512, 400
    sc = Scenario(20, 3, 32, 128, "bf16", seed=59)
    sc.prompt(0, 0)
    sc.append(0, S)
    # plant the values in the pool on both sides (same bits)
    blk, row = sc.ora.block_table(0)[p // 32], p % 32
    for h, d, val in ((1, 7, 65280.0), (2, 100, -65280.0), (0, 5, 65536.0)):
        bits = np.array([val], dtype=np.float32)
        b16 = torch.from_numpy(bits).to(torch.bfloat16)
        assert float(b16[0]) == val
        sc.ov[blk, h, row, d] = b16.view(torch.int16).numpy().view(np.uint16)[0]
        sc.pool.v_cache[blk, h, row, d] = b16[0].cuda()
    sc.check_pool_bits()
    qsl = np.array([0, S], dtype=np.int32)
    q_dev, q64 = sc.random_q(S, "bf16")
    scale = 1 / math.sqrt(128)
    tables, lens = sc.oracle_tables([0])
    ref = A.prefill_chunk(q64, qsl, sc.ok, sc.ov, "bf16", tables, lens, 32, scale)
    got = _run(sc, [0], qsl, q_dev, scale)
    # inside the range: exact up to the weights' fp16 rounding
    for h, d in ((1, 7), (2, 100)):
        col_err = np.abs(got[:, h, d] - ref[:, h, d]).max()
        assert col_err <= 5e-3 * np.abs(ref[:, h, d]).max(), f"head {h} dim {d}: {col_err:.3e}"
    keep = np.ones(got.shape, dtype=bool)
    keep[:, 1, 7] = keep[:, 2, 100] = False
    keep[:, 0, 5] = False
    assert np.all(np.isfinite(got[keep]))
    assert np.abs(got[keep] - ref[keep]).max() <= TOL["bf16"]
    # outside: inf or NaN exactly where the value is seen, exact far before it
    assert not np.any(np.isfinite(got[p:, 0, 5]))
    early = p - 256
    assert np.all(np.isfinite(got[:early, 0, 5]))
    assert np.abs(got[:early, 0, 5] - ref[:early, 0, 5]).max() <= TOL["bf16"]
