"""GPU parity of the cache writes: pa_reshape_and_cache and pa_copy_blocks
against the oracle, bit for bit over the whole pool (every byte outside the
written slots must keep its sentinel)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_166_amd as pa
from oracle import cache as C
from tests.gpu_util import Scenario, bits_to_device, device_bits, to_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [4, 16, 32, 64])
def test_reshape_and_cache_bit_exact(kv, D, bs):
    sc = Scenario(24, 3, bs, D, kv, seed=11)
    rng = np.random.default_rng(12)
    T = 40
    slots = rng.choice(24 * bs, size=T, replace=False).astype(np.int64)
    slots[rng.random(T) < 0.2] = -1                       # skipped rows
    x = to_bits(rng.standard_normal((T, 3, D), dtype=np.float32), kv)
    y = to_bits(rng.standard_normal((T, 3, D), dtype=np.float32), kv)
    pa.pa_reshape_and_cache(sc.pool, bits_to_device(x, kv, "cuda"), bits_to_device(y, kv, "cuda"),
                            torch.from_numpy(slots).cuda())
    C.write_rows(sc.ok, x, slots, bs)
    C.write_rows(sc.ov, y, slots, bs)
    sc.check_pool_bits()


@pytest.mark.parametrize("in_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [8, 32, 64])
def test_reshape_and_cache_fp8_bit_exact(in_dtype, D, bs):
    """Codes are RNE-saturate(x / scale) with the division in float32; the
    scales are chosen so that some values saturate and some are subnormal."""
    sc = Scenario(16, 4, bs, D, "fp8", seed=13, in_dtype=in_dtype, scale_range=(0.002, 0.05))
    rng = np.random.default_rng(14)
    T = 50
    slots = rng.choice(16 * bs, size=T, replace=False).astype(np.int64)
    slots[:3] = -1
    x32 = rng.standard_normal((T, 4, D), dtype=np.float32) * rng.choice([1e-3, 1.0, 3.0], (T, 4, 1))
    x = to_bits(x32.astype(np.float32), in_dtype)
    y = to_bits((x32 * -0.7).astype(np.float32), in_dtype)
    pa.pa_reshape_and_cache(sc.pool, bits_to_device(x, in_dtype, "cuda"),
                            bits_to_device(y, in_dtype, "cuda"), torch.from_numpy(slots).cuda())
    xf = C.to_float64(x, in_dtype).astype(np.float32)
    yf = C.to_float64(y, in_dtype).astype(np.float32)
    C.write_rows_fp8(sc.ok, xf, slots, sc.oks, bs)
    C.write_rows_fp8(sc.ov, yf, slots, sc.ovs, bs)
    sc.check_pool_bits()


@pytest.mark.parametrize("kv", ["f16", "bf16", "fp8", "f32"])
def test_copy_blocks_bit_exact(kv):
    sc = Scenario(20, 5, 16, 128, kv, seed=15)
    for s in range(4):
        sc.prompt(s, 16 * 3 + s)                # fill some blocks
    pairs = [(sc.ora.block_table(0)[0], 17), (sc.ora.block_table(1)[2], 3),
             (sc.ora.block_table(3)[1], 19)]
    free = set(sc.ora.free)
    pairs = [(s, d) for s, d in pairs if d in free]
    assert pairs
    pa.pa_copy_blocks(sc.pool, torch.tensor(pairs, dtype=torch.int32, device="cuda"))
    C.copy_blocks(sc.ok, pairs, sc.oks)
    C.copy_blocks(sc.ov, pairs, sc.ovs)
    sc.check_pool_bits()


def test_write_then_gather_is_the_logical_sequence():
    """Rows written through the library come back in logical order through
    the block table (gather of the GPU pool == the rows written)."""
    sc = Scenario(12, 2, 4, 64, "f16", seed=16)
    rng = np.random.default_rng(17)
    written = {}
    for s, n in [(0, 7), (1, 3), (2, 9)]:
        slots = sc.alloc.alloc_prompt(s, n)
        sc.ora.alloc_prompt(s, n)
        x = to_bits(rng.standard_normal((n, 2, 64), dtype=np.float32), "f16")
        pa.pa_reshape_and_cache(sc.pool, bits_to_device(x, "f16", "cuda"),
                                bits_to_device(x, "f16", "cuda"), torch.from_numpy(slots).cuda())
        written[s] = x
    torch.cuda.synchronize()
    kb = device_bits(sc.pool.k_cache)
    for s, x in written.items():
        assert np.array_equal(C.gather(kb, sc.alloc.block_table(s), sc.alloc.seq_len(s), 4), x)
