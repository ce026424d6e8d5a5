"""Oracle cache write, block copy and gather (test infrastructure only).

The physical pool is one array per K and per V with layout
``[num_blocks, num_heads, block_size, head_dim]`` (a documented choice: the
PagedAttention blog article, section 3.2.1, uses ``[num_blocks, block_size,
num_heads, head_dim]``; the DataWhale notes' exercise has no head axis.  The
gathered result does not depend on the layout, only the indexing below does).

Storage is kept as raw bit patterns so that cache writes can be compared bit
for bit:  float32 -> uint32, float16 / bfloat16 -> uint16, fp8 -> uint8.

* Slot mapping: position p of a sequence lives in physical slot
  ``table[p // bs] * bs + p % bs`` (vLLM course ch. 4, attention pseudocode:
  the block table maps the logical block to the physical block, the token's
  offset inside the block is kept).  A negative slot means "skip".
* Gather: concatenate the table's blocks in order and keep the first L rows
  (DataWhale notes, ``get_physical_cache``; blog article section 3.2.2, the
  key/value collection loop that stops at an invalid (-1) entry).
* Copy-on-write copy: the whole block, K and V, from src to dst (DataWhale
  notes section 4: a new physical block once the sharers diverge; its
  contents start as the shared block's).
"""
import numpy as np

from . import fp8

F32, F16, BF16, FP8 = "f32", "f16", "bf16", "fp8"

_BITS = {F32: np.uint32, F16: np.uint16, BF16: np.uint16, FP8: np.uint8}


def bits_dtype(dt):
    return _BITS[dt]


def to_float64(bits, dt):
    """Exact value of stored bits (fp8 codes are returned unscaled)."""
    bits = np.asarray(bits)
    if dt == F32:
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dt == F16:
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if dt == BF16:
        # bfloat16 is the top half of a float32
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dt == FP8:
        return fp8.decode(bits)
    raise ValueError(dt)


def slot_of(table, pos, block_size):
    return table[pos // block_size] * block_size + pos % block_size


def slot_mapping(table, start, stop, block_size):
    return [slot_of(table, p, block_size) for p in range(start, stop)]


def write_rows(cache_bits, x_bits, slots, block_size):
    """cache[slot // bs, :, slot % bs, :] = x[t] for each token t with slot >= 0.

    cache_bits: [N, H, bs, D]; x_bits: [T, H, D] of the same bit type.
    Slots of one call are distinct.
    """
    slots = np.asarray(slots, dtype=np.int64)
    t = np.nonzero(slots >= 0)[0]
    s = slots[t]
    cache_bits[s // block_size, :, s % block_size, :] = np.asarray(x_bits)[t]
    return cache_bits


def write_rows_fp8(cache_codes, x_f32, slots, scales, block_size):
    """fp8 store: code = RNE-saturate(x / scale[block, head]), x in float32.

    cache_codes: [N, H, bs, D] uint8; x_f32: [T, H, D] float32 values;
    scales: [N, H] float32, the block's existing scale.  Slots are distinct.
    """
    slots = np.asarray(slots, dtype=np.int64)
    t = np.nonzero(slots >= 0)[0]
    s = slots[t]
    blk, off = s // block_size, s % block_size
    codes = fp8.quantize_f32(np.asarray(x_f32, dtype=np.float32)[t], scales[blk][:, :, None])
    cache_codes[blk, :, off, :] = codes
    return cache_codes


def copy_blocks(cache_bits, pairs, scales=None):
    """Whole-block copy for each (src, dst) pair, in order; scales move too."""
    for src, dst in pairs:
        cache_bits[dst] = cache_bits[src]
        if scales is not None:
            scales[dst] = scales[src]
    return cache_bits


def gather(cache_bits, table, length, block_size):
    """Blocks of the table in order, concatenated on the token axis, first L rows.

    Returns [L, H, D] bits.  Only the first ceil(L / bs) table entries are read.
    """
    n = -(-length // block_size)
    if n == 0:
        shape = (0, cache_bits.shape[1], cache_bits.shape[3])
        return np.zeros(shape, dtype=cache_bits.dtype)
    blocks = [cache_bits[table[j]] for j in range(n)]              # each [H, bs, D]
    seq = np.concatenate([b.transpose(1, 0, 2) for b in blocks], axis=0)  # [n*bs, H, D]
    return seq[:length]


def gather_scales(scales, table, length, block_size):
    """Per-token scale [L, H]: the scale of the block holding the token."""
    rows = []
    for p in range(length):
        rows.append(scales[table[p // block_size]])
    if not rows:
        return np.zeros((0, scales.shape[1]), dtype=np.float64)
    return np.asarray(rows, dtype=np.float64)


def write_runs(slots, block_size):
    """Split a call's tokens into runs: maximal groups of consecutive tokens
    whose slots are consecutive positions of one block.  Returns a list of
    (block, first position, [token indices])."""
    slots = np.asarray(slots, dtype=np.int64)
    runs = []
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, pos = int(s // block_size), int(s % block_size)
        if runs and runs[-1][0] == blk and slots[runs[-1][2][-1]] == s - 1 and runs[-1][2][-1] == t - 1:
            runs[-1][2].append(t)
        else:
            runs.append((blk, pos, [t]))
    return runs


def write_rows_fp8_upkeep(cache_codes, x_f32, slots, scales, block_size):
    """fp8 store that keeps each (block, head) scale at amax / 448 of the rows
    the block holds (reading of the blog article's mixed-precision KV, section
    2.3, for blocks that fill a few tokens at a time).

    For each run of the call (one block, consecutive positions p0 ..), and
    each head, in float32:
      s_run = amax(|x| over the run's rows) / 448;
      s_old = 0 if the run starts the block (p0 == 0) else scales[block, head];
      s_new = max(s_old, s_run);
      if s_new > s_old and p0 > 0, the block's earlier rows 0 .. p0-1 are
      requantised: code' = RNE-saturate((decode(code) * s_old) / s_new);
      the run's rows are stored as RNE-saturate(x / s_new);
      scales[block, head] = s_new.
    While a block's scale is 0 (every value so far zero) the divisor is 1, so
    zeros keep their sign.  Each block's new rows must form one run of the
    call, at positions after the rows it already holds (what the allocator's
    slot mappings give).  cache_codes [N, H, bs, D] uint8, x_f32 [T, H, D],
    scales [N, H] float32, all updated in place.
    """
    x = np.asarray(x_f32, dtype=np.float32)
    f448 = np.float32(fp8.MAX_FINITE)
    runs = write_runs(slots, block_size)
    blocks = [r[0] for r in runs]
    if len(set(blocks)) != len(blocks):
        raise ValueError("a block's new rows must form one run of the call")
    for blk, p0, toks in runs:
        rows = x[toks]                                     # [n, H, D]
        n = len(toks)
        for h in range(cache_codes.shape[1]):
            s_run = np.float32(np.abs(rows[:, h, :]).max()) / f448
            s_old = np.float32(0.0) if p0 == 0 else np.float32(scales[blk, h])
            s_new = max(s_old, s_run)
            div_new = s_new if s_new > 0 else np.float32(1.0)
            if p0 > 0 and s_new > s_old:
                old = cache_codes[blk, h, :p0, :]
                v = fp8.decode(old).astype(np.float32) * s_old   # float32 product
                cache_codes[blk, h, :p0, :] = fp8.quantize_f32(v, div_new)
            cache_codes[blk, h, p0:p0 + n, :] = fp8.quantize_f32(rows[:, h, :], div_new)
            scales[blk, h] = s_new
    return cache_codes
