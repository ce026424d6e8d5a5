"""Plain CPU oracle for paged attention over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
anything from this package.  The GPU library (``paged_kv_cache_166_amd``)
never imports it and it never imports the GPU library: the two share no
kernels, headers, helpers, tables or constants.

What it computes, and where the pages define it:

* ``allocator`` -- the block manager: a free list of fixed-size physical
  blocks, ceil(len / block_size) blocks for a prompt, one more block when a
  decode step crosses a block boundary, an out-of-memory error when the free
  list runs short, blocks returned on free, and copy-on-write sharing of
  prefix blocks.  ("vLLM PagedAttention" study notes, KVCacheManager exercise
  and the copy-on-write paragraph of section 4; vLLM tuning course ch. 4,
  "Block management strategy" table and allocation flow.)
* ``cache`` -- slot mapping, the cache write, the whole-block copy used by
  copy-on-write, and the gather of a sequence's blocks into one contiguous
  K/V.  (Study notes, ``get_physical_cache``; course ch. 4 attention
  pseudocode.)
* ``attention`` -- textbook softmax attention in float64 over the gathered
  K/V, for one decode token per sequence and for a causal query chunk.
  (PagedAttention blog article, section 3.2.2 forward pass; course ch. 4.)
* ``fp8`` -- the OCP FP8 E4M3FN codec written from the format definition.

Every function is written for readability, not speed.  Pins that tie each
function to the pages or to mathematics live in ``tests/test_oracle_*.py``.
The only part without a printed worked example is the attention arithmetic;
it is pinned by closed forms, an independent library routine and brute force.
"""
