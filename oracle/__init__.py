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
* ``fp8`` -- the OCP FP8 E4M3FN codec written from the format definition;
  ``cache`` also holds the fp8 write with per-(block, head) scale upkeep
  (the blog's mixed-precision KV storage).
* ``prefix`` -- the prefix index over token ids as a flat list with
  longest-common-prefix matching, bound to the allocator (study notes,
  RadixAttention section and its exercise).
* ``radix`` -- the same index as a radix tree, with least-recently-used
  eviction of leaves when memory runs out (study notes, same section).
* ``buddy`` -- a block size per request carved from one arena by a binary
  buddy system (blog, "3.0" feature list: a page size fitted to the
  request's length).

Every function is written for readability, not speed.  Pins that tie each
function to the pages or to mathematics live in ``tests/test_oracle_*.py``.
The attention arithmetic has no printed worked example; it is pinned by
closed forms, an independent library routine and brute force.  The eviction
and buddy readings are pinned by hand-worked cases and invariants.
"""
