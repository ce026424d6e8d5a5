"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module holds no part of the attention or allocation arithmetic: it only
names the configurations, draws lengths, permutations and normal random
values, and lists call sequences.  Both the GPU library's callers and the CPU
oracle's callers take their inputs from here.

Configurations (sizes are those of the workloads the pages discuss: 16- and
32-token blocks, LLaMA-13B-shaped heads, long contexts, shared prefixes):

* ``tiny_decode``      3 sequences of 6, 9, 5 tokens, block 4, pool of 10
                        shuffled, 4 heads x 64, fp32, plus a 1-block OOM case.
* ``llama13b_decode``  32 sequences, 40 heads x 128, fp16, block 16,
                        lengths uniform in [128, 2048], pool of 4096 shuffled.
* ``prefix_cow``       64 sequences sharing a 1024-token prefix plus 1..256
                        distinct tokens, 40 x 128, bf16, block 16, pool 4096.
* ``chunked_prefill``  8 sequences, a 512-token chunk after 0..3584 tokens of
                        context, 32 x 128, bf16, block 32, pool 4096.
* ``long_fp8_decode``  4 sequences of 131072 tokens, 32 x 128, block 32,
                        fp8 E4M3 KV with a float32 scale per (block, head),
                        bf16 query, 256 partitions, pool 16384 shuffled.
"""
import numpy as np

CONFIGS = {
    "tiny_decode": dict(batch=3, lens=(6, 9, 5), block_size=4, num_blocks=10, num_heads=4,
                        head_dim=64, kv_dtype="f32", q_dtype="f32", seed=1),
    "llama13b_decode": dict(batch=32, num_heads=40, head_dim=128, kv_dtype="f16", q_dtype="f16",
                            block_size=16, len_lo=128, len_hi=2048, num_blocks=4096, seed=2),
    "prefix_cow": dict(batch=64, prefix=1024, suffix_lo=1, suffix_hi=256, num_heads=40,
                       head_dim=128, kv_dtype="bf16", q_dtype="bf16", block_size=16,
                       num_blocks=4096, seed=3),
    "chunked_prefill": dict(batch=8, chunk=512, ctx_lo=0, ctx_hi=3584, num_heads=32, head_dim=128,
                            kv_dtype="bf16", q_dtype="bf16", block_size=32, num_blocks=4096, seed=4),
    "long_fp8_decode": dict(batch=4, context=131072, num_heads=32, head_dim=128, kv_dtype="fp8",
                            q_dtype="bf16", block_size=32, num_blocks=16384, partitions=256,
                            partition_blocks=16, seed=5),
}


def rng(seed):
    return np.random.default_rng(seed)


def free_order(seed, num_blocks):
    """Initial free-list order: a seeded permutation of the block ids."""
    return rng(seed).permutation(num_blocks).astype(np.int32)


def uniform_ints(seed, n, lo, hi, salt=0):
    """n integers uniform in [lo, hi] inclusive."""
    return rng(seed * 1000 + 17 + salt).integers(lo, hi + 1, size=n).astype(np.int64)


def normal_f32(seed, shape, salt=0):
    """float32 N(0, 1) values (host)."""
    return rng(seed * 7919 + 101 + salt).standard_normal(shape, dtype=np.float32)


def tiny_decode_ops():
    """Call sequence of the tiny decode case: three prompts, then decode steps.

    Sequence ids 0, 1, 2 end with 6, 9 and 5 tokens; sequence 2 crosses the
    4 -> 5 block boundary.  Each op is ("prompt", seq, n) or ("append", seq, 1).
    """
    return [("prompt", 0, 6), ("prompt", 1, 6), ("prompt", 2, 4),
            ("append", 1, 1), ("append", 2, 1), ("append", 1, 1), ("append", 1, 1)]


def torch_normal(shape, seed, device, dtype):
    """Seeded N(0, 1) tensor generated where it will live, then cast (RNE)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)
