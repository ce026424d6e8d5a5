"""GPU parity of the fp8 write with scale upkeep (PA_POOL_FP8_AUTO_SCALE):
codes and per-(block, head) scales bit for bit against the oracle after every
call -- decode-style appends that grow, keep and shrink the amplitude across
block boundaries, chunk writes that requantise a partly filled block, zero
rows, stale scales left in freshly allocated blocks -- then pa_decode over the
auto-scaled pool against the oracle at the fp8 tolerance."""
import math

import numpy as np
import pytest

from tests.gpu_util import TOL, Scenario, assert_close
from tests.test_gpu_decode import _oracle, _run_decode

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("in_dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D,bs", [(128, 16), (64, 4), (128, 32), (128, 64), (64, 64)])
def test_appends_grow_keep_and_shrink(in_dtype, D, bs):
    H = 3
    # stale scales (50..100) in every block: a run that starts a block must ignore them
    sc = Scenario(64, H, bs, D, "fp8", seed=40 + D + bs, in_dtype=in_dtype,
                  scale_range=(50.0, 100.0), fp8_auto_scale=True)
    rng = np.random.default_rng(D + bs)
    lens = [1, bs - 1 if bs > 1 else 1, bs + 3, 2 * bs]
    for i, L in enumerate(lens):
        sc.prompt(i, L, amp=rng.uniform(0.1, 4.0, (L, H, 1)))
    sc.check_pool_bits()
    seqs = list(range(len(lens)))
    for step in range(2 * bs + 3):
        amp = rng.choice([0.05, 1.0, 30.0], size=(len(seqs), H, 1))
        sc.write_batch(seqs, 1, amp)
        sc.check_pool_bits()


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bs", [32, 64])
def test_chunks_requantise_the_partly_filled_block(in_dtype, bs):
    H, D = 4, 128
    sc = Scenario(200, H, bs, D, "fp8", seed=77, in_dtype=in_dtype, fp8_auto_scale=True)
    rng = np.random.default_rng(77)
    for i, (L, a) in enumerate([(10, 0.5), (40, 2.0), (33, 1.0), (64, 0.01)]):
        sc.prompt(i, L, amp=a)
    sc.check_pool_bits()
    seqs = [0, 1, 2, 3]
    sc.write_batch(seqs, 50, amp=rng.uniform(0.1, 10.0, (4 * 50, H, 1)))   # one call, runs per block
    sc.check_pool_bits()
    sc.write_batch(seqs, 5, amp=0.0)                                       # signed zeros
    sc.check_pool_bits()
    sc.write_batch(seqs, 70, amp=rng.uniform(0.1, 100.0, (4 * 70, H, 1)))
    sc.check_pool_bits()


def test_all_zero_block_keeps_zero_scale_then_grows():
    sc = Scenario(16, 2, 8, 64, "fp8", seed=5, in_dtype="bf16", fp8_auto_scale=True)
    sc.prompt(0, 3, amp=0.0)
    sc.check_pool_bits()
    assert np.all(sc.oks[sc.ora.block_table(0)[0]] == 0.0)
    sc.append(0, 2, amp=1.5)
    sc.check_pool_bits()


def test_decode_over_an_auto_scaled_pool():
    H, D, bs = 4, 128, 16
    sc = Scenario(300, H, bs, D, "fp8", seed=91, in_dtype="bf16", fp8_auto_scale=True)
    rng = np.random.default_rng(91)
    lens = [1, 17, 130, 511, 700]
    for i, L in enumerate(lens):
        sc.prompt(i, L, amp=rng.uniform(0.5, 2.0, (L, H, 1)))
    seqs = list(range(len(lens)))
    for _ in range(20):
        sc.write_batch(seqs, 1, rng.choice([0.5, 1.0, 3.0], size=(len(seqs), H, 1)))
    sc.check_pool_bits()
    q_dev, q64 = sc.random_q(len(seqs), "bf16")
    scale = 1 / math.sqrt(D)
    ref = _oracle(sc, seqs, q64, scale)
    for pb in (0, 3):
        got, _, _ = _run_decode(sc, seqs, q_dev, scale, pb)
        assert_close(got, ref, TOL["fp8"], f"auto-scaled fp8 pb={pb}")


def test_a_large_mixed_call():
    """Over 1024 tokens in one call (the kernel then gives each wave a window
    of one block of tokens): long chunks starting mid-block next to one-token
    runs, so windows hold several run heads and runs cross window edges."""
    H, D, bs = 2, 128, 16
    sc = Scenario(400, H, bs, D, "fp8", seed=123, in_dtype="bf16", fp8_auto_scale=True,
                  scale_range=(50.0, 100.0))
    rng = np.random.default_rng(123)
    lens = [5, 16, 1, 37, 9, 3]
    for i, L in enumerate(lens):
        sc.prompt(i, L, amp=rng.uniform(0.1, 2.0, (L, H, 1)))
    seqs = list(range(len(lens)))
    ns = [500, 1, 300, 1, 420, 2]
    sc.write_batch(seqs, ns, amp=rng.uniform(0.1, 20.0, (sum(ns), H, 1)))
    sc.check_pool_bits()
    sc.write_batch(seqs, [1, 700, 1, 400, 1, 3], amp=rng.uniform(0.1, 50.0, (1106, H, 1)))
    sc.check_pool_bits()
