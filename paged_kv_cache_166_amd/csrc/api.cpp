// C ABI of the GPU calls in pa.h: argument checks, then one launch each.
// Nothing is launched when a check fails.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "kernels.h"
#include "pa.h"
#include "status.h"

namespace {

using pa::fail;

bool valid_dtype(int32_t dt) { return dt >= PA_F32 && dt <= PA_FP8_E4M3; }
bool valid_io_dtype(int32_t dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int elem_bytes(int32_t dt) { return dt == PA_F32 ? 4 : (dt == PA_FP8_E4M3 ? 1 : 2); }

pa_status check_pool(const char* fn, const pa_pool* p) {
  if (!p) return fail(PA_ERR_INVALID, "%s: pool is NULL", fn);
  if (!p->k_cache || !p->v_cache) return fail(PA_ERR_INVALID, "%s: NULL cache pointer", fn);
  if (!aligned(p->k_cache, 128) || !aligned(p->v_cache, 128))
    return fail(PA_ERR_INVALID, "%s: cache bases must be 128-byte aligned", fn);
  if (p->num_blocks <= 0 || p->num_heads <= 0 || p->num_heads > 65535)
    return fail(PA_ERR_INVALID, "%s: num_blocks=%d num_heads=%d", fn, p->num_blocks, p->num_heads);
  if (p->block_size != 4 && p->block_size != 8 && p->block_size != 16 && p->block_size != 32 &&
      p->block_size != 64)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (built: 4, 8, 16, 32, 64)", fn,
                p->block_size);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (built: 64, 128)", fn, p->head_dim);
  if (!valid_dtype(p->kv_dtype)) return fail(PA_ERR_INVALID, "%s: kv_dtype %d", fn, p->kv_dtype);
  if (p->flags & ~(PA_POOL_STREAM_KV | PA_POOL_FP8_AUTO_SCALE))
    return fail(PA_ERR_INVALID, "%s: unknown pool flags 0x%x", fn, p->flags);
  if ((p->flags & PA_POOL_FP8_AUTO_SCALE) && p->kv_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_INVALID, "%s: PA_POOL_FP8_AUTO_SCALE on a pool that is not fp8", fn);
  if (p->kv_dtype == PA_FP8_E4M3) {
    if (!p->k_scale || !p->v_scale) return fail(PA_ERR_INVALID, "%s: fp8 pool without scales", fn);
  }
  return PA_OK;
}

// A table row addresses at most INT32_MAX tokens (context lengths are
// int32); a wider row would overflow the partition arithmetic below.
bool row_fits(const pa_pool* p, int32_t max_blocks) {
  return max_blocks > 0 && int64_t(max_blocks) * p->block_size <= INT32_MAX;
}

pa_status hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return PA_OK;
}

// Partitions per sequence are the launch grid's z dimension.
constexpr int32_t kMaxParts = 65535;

// 512 tokens per partition: long enough that a workgroup's fixed costs
// (table and query loads, the final merge) are small next to its stream of
// K/V, short enough that ragged batches still split into many workgroups.
int32_t auto_partition_blocks(const pa_pool* p) {
  int32_t b = 512 / p->block_size;
  return b < 1 ? 1 : (b > 256 ? 256 : b);
}

struct WsLayout {
  int64_t ml_off, acc_off, bytes;
  int32_t parts;
};

WsLayout ws_layout_parts(const pa_pool* p, int32_t num_seqs, int32_t parts) {
  WsLayout w{};
  w.parts = parts;
  if (w.parts <= 1) return w;
  const int64_t sh = int64_t(num_seqs) * p->num_heads;
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  w.ml_off = 0;
  w.acc_off = up(sh * w.parts * 2 * 4);
  w.bytes = w.acc_off + up(sh * w.parts * p->head_dim * 4);
  return w;
}

// The shared-prefix decode's geometry: prefix chunks (whole 32-key tiles,
// at least 256 keys, at most about 64 chunks) and suffix partitions.  A
// chunk's workgroup costs about the same from 4 to 8 tiles (its fixed
// latency dominates), while each chunk adds a partial per (sequence, head).
struct PrefixPlan {
  int32_t prefix_len, chunk_keys, chunks, suffix_pb, suffix_parts, total_parts;
};

PrefixPlan prefix_plan(const pa_pool* p, int32_t max_blocks, int32_t shared_blocks,
                       int32_t partition_blocks) {
  PrefixPlan g{};
  g.prefix_len = shared_blocks * p->block_size;
  const int32_t want = int32_t((int64_t(g.prefix_len) + 63) / 64);
  g.chunk_keys = std::max<int32_t>(256, (want + 31) / 32 * 32);
  g.chunks = (g.prefix_len + g.chunk_keys - 1) / g.chunk_keys;
  g.suffix_pb = partition_blocks > 0 ? partition_blocks : auto_partition_blocks(p);
  g.suffix_parts = (max_blocks - shared_blocks + g.suffix_pb - 1) / g.suffix_pb;
  g.total_parts = g.chunks + g.suffix_parts;
  return g;
}

WsLayout ws_layout(const pa_pool* p, int32_t num_seqs, int32_t max_blocks, int32_t part_blocks) {
  return ws_layout_parts(p, num_seqs, (max_blocks + part_blocks - 1) / part_blocks);
}

// The several-pool decode: pools agree on heads, head_dim, KV type; every
// group's block size divides the partition length; partitions per sequence
// at most ceil(max_blocks * block_size / part_tokens) over the groups.
pa_status check_multi(const char* fn, const pa_pool* pools, int32_t num_groups,
                      const int32_t* max_blocks, int32_t part_tokens, int32_t* parts) {
  if (!pools || !max_blocks || num_groups < 1 || num_groups > pa::kMaxDecodeGroups)
    return fail(PA_ERR_INVALID, "%s: 1..%d groups with pools and table widths", fn,
                pa::kMaxDecodeGroups);
  *parts = 1;
  for (int32_t g = 0; g < num_groups; ++g) {
    if (pa_status st = check_pool(fn, &pools[g])) return st;
    if (pools[g].num_heads != pools[0].num_heads || pools[g].head_dim != pools[0].head_dim ||
        pools[g].kv_dtype != pools[0].kv_dtype)
      return fail(PA_ERR_INVALID, "%s: pools differ in heads, head_dim or KV type", fn);
    const int32_t bs = pools[g].block_size;
    if (part_tokens % bs != 0 || part_tokens / bs > 256)
      return fail(PA_ERR_UNSUPPORTED,
                  "%s: partition of %d tokens is not 1..256 blocks of %d", fn, part_tokens, bs);
    if (!row_fits(&pools[g], max_blocks[g]))
      return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq %d (1..INT32_MAX / block_size)", fn,
                  max_blocks[g]);
    const int64_t p = (int64_t(max_blocks[g]) * bs + part_tokens - 1) / part_tokens;
    if (p > kMaxParts)
      return fail(PA_ERR_UNSUPPORTED, "%s: %lld partitions per sequence (at most %d)", fn,
                  (long long)p, kMaxParts);
    *parts = std::max<int32_t>(*parts, int32_t(p));
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_reshape_and_cache(const pa_pool* pool, const void* key, const void* value,
                               int32_t in_dtype, const int64_t* slot_mapping,
                               int32_t num_tokens, hipStream_t stream) {
  const char* fn = "pa_reshape_and_cache";
  if (pa_status s = check_pool(fn, pool)) return s;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "%s: num_tokens < 0", fn);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID, "%s: key/value must be 16-byte aligned", fn);
  if (pool->kv_dtype == PA_FP8_E4M3) {
    if (!valid_io_dtype(in_dtype))
      return fail(PA_ERR_INVALID, "%s: fp8 pool takes f32/f16/bf16 rows, got %d", fn, in_dtype);
  } else if (in_dtype != pool->kv_dtype) {
    return fail(PA_ERR_INVALID, "%s: in_dtype %d must equal kv_dtype %d", fn, in_dtype,
                pool->kv_dtype);
  }
  pa::CacheWriteArgs a{pool->k_cache, pool->v_cache, pool->k_scale, pool->v_scale,
                       key,           value,         slot_mapping,  num_tokens,
                       pool->num_heads, pool->block_size, pool->head_dim, in_dtype,
                       pool->kv_dtype,  (pool->flags & PA_POOL_FP8_AUTO_SCALE) != 0};
  return hip_status(fn, pa::launch_reshape_and_cache(a, stream));
}

pa_status pa_copy_blocks(const pa_pool* pool, const int32_t* src_dst, int32_t num_pairs,
                         hipStream_t stream) {
  const char* fn = "pa_copy_blocks";
  if (pa_status s = check_pool(fn, pool)) return s;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "%s: num_pairs < 0", fn);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_ERR_INVALID, "%s: src_dst is NULL", fn);
  const bool fp8 = pool->kv_dtype == PA_FP8_E4M3;
  pa::CopyBlocksArgs a{pool->k_cache,
                       pool->v_cache,
                       fp8 ? pool->k_scale : nullptr,
                       fp8 ? pool->v_scale : nullptr,
                       src_dst,
                       num_pairs,
                       pool->num_heads,
                       int64_t(pool->block_size) * pool->head_dim * elem_bytes(pool->kv_dtype)};
  return hip_status(fn, pa::launch_copy_blocks(a, stream));
}

int32_t pa_decode_auto_partition_blocks(const pa_pool* pool, int32_t num_seqs,
                                        int32_t max_blocks_per_seq) {
  (void)num_seqs;
  (void)max_blocks_per_seq;
  if (check_pool("pa_decode_auto_partition_blocks", pool)) return -1;
  return auto_partition_blocks(pool);
}

size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, int32_t partition_blocks) {
  if (check_pool("pa_decode_workspace_bytes", pool)) return 0;
  if (num_seqs <= 0 || !row_fits(pool, max_blocks_per_seq) || partition_blocks < 0 ||
      partition_blocks > 256)
    return 0;
  const int32_t pb = partition_blocks > 0 ? partition_blocks : auto_partition_blocks(pool);
  return size_t(ws_layout(pool, num_seqs, max_blocks_per_seq, pb).bytes);
}

}  // extern "C"

namespace {

// pa_decode, and pa_decode_append when key_new is not NULL.
pa_status decode_impl(const char* fn, void* out, int32_t out_dtype, const void* q,
                      int32_t q_dtype, const pa_pool* pool, const void* key_new,
                      const void* value_new, const int64_t* new_slots,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, float scale,
                      int32_t partition_blocks, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (pa_status s = check_pool(fn, pool)) return s;
  if (num_seqs < 0 || num_seqs > 65535) return fail(PA_ERR_INVALID, "%s: num_seqs %d", fn, num_seqs);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID, "%s: q and out must be 16-byte aligned", fn);
  if (!row_fits(pool, max_blocks_per_seq))
    return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq %d (1..INT32_MAX / block_size)", fn,
                max_blocks_per_seq);
  if (pool->kv_dtype == PA_FP8_E4M3) {
    if (!valid_io_dtype(q_dtype)) return fail(PA_ERR_INVALID, "%s: q_dtype %d", fn, q_dtype);
  } else if (q_dtype != pool->kv_dtype) {
    return fail(PA_ERR_UNSUPPORTED, "%s: q_dtype %d must equal kv_dtype %d", fn, q_dtype,
                pool->kv_dtype);
  }
  if (out_dtype != PA_F32 && out_dtype != q_dtype)
    return fail(PA_ERR_INVALID, "%s: out_dtype must be f32 or q_dtype", fn);
  if (partition_blocks < 0 || partition_blocks > 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: partition_blocks %d (1..256, or 0 = auto)", fn,
                partition_blocks);
  const int32_t pb = partition_blocks > 0 ? partition_blocks : auto_partition_blocks(pool);
  const WsLayout w = ws_layout(pool, num_seqs, max_blocks_per_seq, pb);
  if (w.parts > kMaxParts)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d partitions per sequence (at most %d)", fn, w.parts,
                kMaxParts);
  if (w.parts > 1) {
    if (!workspace || size_t(w.bytes) > workspace_bytes || !aligned(workspace, 256))
      return fail(PA_ERR_INVALID, "%s: workspace of %lld bytes, 256-byte aligned, is required",
                  fn, (long long)w.bytes);
  }
  char* ws = static_cast<char*>(workspace);
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws_ml = w.parts > 1 ? reinterpret_cast<float*>(ws + w.ml_off) : nullptr;
  a.ws_acc = w.parts > 1 ? reinterpret_cast<float*>(ws + w.acc_off) : nullptr;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = pool->num_heads;
  a.block_size = pool->block_size;
  a.part_blocks = pb;
  a.max_parts = w.parts < 1 ? 1 : w.parts;
  a.ws_parts = a.max_parts;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.q_dtype = q_dtype;
  a.out_dtype = out_dtype;
  if (key_new) {
    if (!value_new || !new_slots) return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
    if (!aligned(key_new, 16) || !aligned(value_new, 16) || !aligned(new_slots, 8))
      return fail(PA_ERR_INVALID, "%s: key_new/value_new must be 16-byte aligned", fn);
    a.k_new = key_new;
    a.v_new = value_new;
    a.new_slots = new_slots;
    a.fp8_upkeep = (pool->flags & PA_POOL_FP8_AUTO_SCALE) != 0;
  }
  return hip_status(fn, pa::launch_decode(a, pool->kv_dtype, pool->head_dim, pool->block_size,
                                          (pool->flags & PA_POOL_STREAM_KV) != 0, num_seqs,
                                          stream));
}

}  // namespace

extern "C" {

pa_status pa_decode(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                    const pa_pool* pool, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    float scale, int32_t partition_blocks, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return decode_impl("pa_decode", out, out_dtype, q, q_dtype, pool, nullptr, nullptr, nullptr,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, scale,
                     partition_blocks, workspace, workspace_bytes, stream);
}

pa_status pa_decode_noalloc(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                            const pa_pool* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, float scale, int32_t partition_blocks,
                            hipStream_t stream) {
  const char* fn = "pa_decode_noalloc";
  if (pa_status s = check_pool(fn, pool)) return s;
  // Size first (no HIP call before it): a batch the array cannot hold is
  // refused outright.  Arguments pa_decode would refuse give 0 here and are
  // refused by decode_impl below.
  const size_t need =
      pa_decode_workspace_bytes(pool, num_seqs, max_blocks_per_seq, partition_blocks);
  if (need > PA_DECODE_NOALLOC_MAX_WORKSPACE)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: this batch needs %zu bytes of split-K scratch, more than the %u of the "
                "fixed array; use pa_decode with a workspace",
                fn, need, PA_DECODE_NOALLOC_MAX_WORKSPACE);
  void* ws = nullptr;
  if (need > 0 && num_seqs > 0) {
    if (pa_status s = hip_status(fn, pa::noalloc_scratch(stream, &ws))) return s;
  }
  return decode_impl(fn, out, out_dtype, q, q_dtype, pool, nullptr, nullptr, nullptr,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, scale,
                     partition_blocks, ws, need > 0 ? size_t(PA_DECODE_NOALLOC_MAX_WORKSPACE) : 0,
                     stream);
}

pa_status pa_decode_append(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                           const pa_pool* pool, const void* key_new, const void* value_new,
                           const int64_t* new_slots, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, float scale, int32_t partition_blocks,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!key_new) return fail(PA_ERR_INVALID, "pa_decode_append: key_new is NULL");
  return decode_impl("pa_decode_append", out, out_dtype, q, q_dtype, pool, key_new, value_new,
                     new_slots, block_tables, max_blocks_per_seq, context_lens, num_seqs, scale,
                     partition_blocks, workspace, workspace_bytes, stream);
}

size_t pa_decode_shared_prefix_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                               int32_t max_blocks_per_seq, int32_t shared_blocks,
                                               int32_t partition_blocks) {
  if (check_pool("pa_decode_shared_prefix_workspace_bytes", pool)) return 0;
  if (num_seqs <= 0 || !row_fits(pool, max_blocks_per_seq) || shared_blocks <= 0 ||
      shared_blocks > max_blocks_per_seq || partition_blocks < 0 || partition_blocks > 256)
    return 0;
  const PrefixPlan g = prefix_plan(pool, max_blocks_per_seq, shared_blocks, partition_blocks);
  // always a workspace: the prefix's partials are merged even alone
  return size_t(ws_layout_parts(pool, num_seqs, std::max(g.total_parts, 2)).bytes);
}

}  // extern "C"

namespace {

// pa_decode_shared_prefix, and pa_decode_shared_prefix_append when key_new
// is not NULL.
pa_status shared_prefix_impl(const char* fn, void* out, int32_t out_dtype, const void* q,
                             int32_t q_dtype, const pa_pool* pool, const void* key_new,
                             const void* value_new, const int64_t* new_slots,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t shared_blocks, float scale, int32_t partition_blocks,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (pa_status st = check_pool(fn, pool)) return st;

  if (num_seqs < 0 || num_seqs > 65535) return fail(PA_ERR_INVALID, "%s: num_seqs %d", fn, num_seqs);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID, "%s: q and out must be 16-byte aligned", fn);
  // the prefix pass runs on MFMA: 16-bit queries (the pool's type, or f16 /
  // bf16 for fp8 pools)
  if (pool->kv_dtype == PA_FP8_E4M3 ? (q_dtype != PA_F16 && q_dtype != PA_BF16)
                                    : q_dtype != pool->kv_dtype)
    return fail(PA_ERR_UNSUPPORTED, "%s: q_dtype %d with kv_dtype %d", fn, q_dtype,
                pool->kv_dtype);
  if (pool->kv_dtype == PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "%s: f32 pools (the prefix pass runs on MFMA)", fn);
  if (out_dtype != PA_F32 && out_dtype != q_dtype)
    return fail(PA_ERR_INVALID, "%s: out_dtype must be f32 or q_dtype", fn);
  if (!row_fits(pool, max_blocks_per_seq))
    return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq %d (1..INT32_MAX / block_size)", fn,
                max_blocks_per_seq);
  if (shared_blocks <= 0 || shared_blocks > max_blocks_per_seq)
    return fail(PA_ERR_INVALID, "%s: shared_blocks %d (1..max_blocks_per_seq %d)", fn,
                shared_blocks, max_blocks_per_seq);
  if (partition_blocks < 0 || partition_blocks > 256)
    return fail(PA_ERR_UNSUPPORTED, "%s: partition_blocks %d (1..256, or 0 = auto)", fn,
                partition_blocks);
  const PrefixPlan g = prefix_plan(pool, max_blocks_per_seq, shared_blocks, partition_blocks);
  if (g.total_parts > kMaxParts)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d partitions per sequence (at most %d)", fn,
                g.total_parts, kMaxParts);
  const WsLayout w = ws_layout_parts(pool, num_seqs, std::max(g.total_parts, 2));
  if (!workspace || size_t(w.bytes) > workspace_bytes || !aligned(workspace, 256))
    return fail(PA_ERR_INVALID, "%s: workspace of %lld bytes, 256-byte aligned, is required", fn,
                (long long)w.bytes);
  if (key_new) {
    if (!value_new || !new_slots) return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
    if (!aligned(key_new, 16) || !aligned(value_new, 16) || !aligned(new_slots, 8))
      return fail(PA_ERR_INVALID, "%s: key_new/value_new must be 16-byte aligned", fn);
  }
  char* ws = static_cast<char*>(workspace);
  float* ws_ml = reinterpret_cast<float*>(ws + w.ml_off);
  float* ws_acc = reinterpret_cast<float*>(ws + w.acc_off);
  const float scale_log2 = scale * 1.4426950408889634f;

  // 1. the shared prefix: every sequence's query against the prefix keys,
  //    chunk by chunk, into partitions 0 .. chunks-1
  pa::PrefillArgs pf{};
  pf.q = q;
  pf.k_cache = pool->k_cache;
  pf.v_cache = pool->v_cache;
  pf.k_scale = pool->k_scale;
  pf.v_scale = pool->v_scale;
  pf.block_tables = block_tables;  // sequence 0's row holds the prefix
  pf.max_blocks_per_seq = max_blocks_per_seq;
  pf.num_heads = pool->num_heads;
  pf.num_seqs = num_seqs;
  pf.scale_log2 = scale_log2;
  pf.out_dtype = out_dtype;
  pf.ws_acc = ws_acc;
  pf.ws_ml = ws_ml;
  pf.max_parts = w.parts;
  pf.prefix_len = g.prefix_len;
  pf.chunk_keys = g.chunk_keys;
  if (pa_status st = hip_status(fn, pa::launch_prefix_partials(pf, pool->kv_dtype, q_dtype, pool->head_dim,
                                                               pool->block_size, stream)))
    return st;

  // 2. each sequence's own blocks after the prefix, into the partitions
  //    after those, then 3. the merge of all of them
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws_ml = ws_ml;
  a.ws_acc = ws_acc;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = pool->num_heads;
  a.block_size = pool->block_size;
  a.part_blocks = g.suffix_pb;
  a.max_parts = std::max(g.suffix_parts, 1);
  a.first_block = shared_blocks;
  a.prefix_parts = g.chunks;
  a.ws_parts = w.parts;
  a.scale_log2 = scale_log2;
  a.q_dtype = q_dtype;
  a.out_dtype = out_dtype;
  // every sequence's own blocks fit one partition: that workgroup merges
  a.fuse_merge = g.suffix_parts <= 1 ? 1 : 0;
  a.k_new = key_new;
  a.v_new = value_new;
  a.new_slots = key_new ? new_slots : nullptr;
  a.fp8_upkeep = (pool->flags & PA_POOL_FP8_AUTO_SCALE) != 0;
  return hip_status(fn, pa::launch_decode(a, pool->kv_dtype, pool->head_dim, pool->block_size,
                                          (pool->flags & PA_POOL_STREAM_KV) != 0, num_seqs,
                                          stream));
}

}  // namespace

extern "C" {

pa_status pa_decode_shared_prefix(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                  const pa_pool* pool, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t shared_blocks, float scale,
                                  int32_t partition_blocks, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return shared_prefix_impl("pa_decode_shared_prefix", out, out_dtype, q, q_dtype, pool, nullptr,
                            nullptr, nullptr, block_tables, max_blocks_per_seq, context_lens,
                            num_seqs, shared_blocks, scale, partition_blocks, workspace,
                            workspace_bytes, stream);
}

pa_status pa_decode_shared_prefix_append(void* out, int32_t out_dtype, const void* q,
                                         int32_t q_dtype, const pa_pool* pool,
                                         const void* key_new, const void* value_new,
                                         const int64_t* new_slots, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t shared_blocks, float scale,
                                         int32_t partition_blocks, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  if (!key_new) return fail(PA_ERR_INVALID, "pa_decode_shared_prefix_append: key_new is NULL");
  return shared_prefix_impl("pa_decode_shared_prefix_append", out, out_dtype, q, q_dtype, pool,
                            key_new, value_new, new_slots, block_tables, max_blocks_per_seq,
                            context_lens, num_seqs, shared_blocks, scale, partition_blocks,
                            workspace, workspace_bytes, stream);
}

size_t pa_decode_multi_workspace_bytes(const pa_pool* pools, const int32_t* max_blocks_per_seq,
                                       int32_t num_groups, int32_t num_seqs,
                                       int32_t partition_tokens) {
  const int32_t pt = partition_tokens > 0 ? partition_tokens : 512;
  int32_t parts = 1;
  if (num_seqs <= 0 ||
      check_multi("pa_decode_multi_workspace_bytes", pools, num_groups, max_blocks_per_seq, pt,
                  &parts))
    return 0;
  return size_t(ws_layout_parts(&pools[0], num_seqs, parts).bytes);
}

pa_status pa_decode_multi(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                          const pa_pool* pools, int32_t num_groups,
                          const int32_t* const* block_tables, const int32_t* max_blocks_per_seq,
                          const int32_t* seq_begin, const int32_t* context_lens, float scale,
                          int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const char* fn = "pa_decode_multi";
  const int32_t pt = partition_tokens > 0 ? partition_tokens : 512;
  if (partition_tokens < 0) return fail(PA_ERR_INVALID, "%s: partition_tokens < 0", fn);
  int32_t parts = 1;
  if (pa_status st = check_multi(fn, pools, num_groups, max_blocks_per_seq, pt, &parts)) return st;
  if (!seq_begin || !block_tables) return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (seq_begin[0] != 0) return fail(PA_ERR_INVALID, "%s: seq_begin[0] must be 0", fn);
  for (int32_t g = 0; g < num_groups; ++g) {
    if (seq_begin[g + 1] < seq_begin[g])
      return fail(PA_ERR_INVALID, "%s: seq_begin must not decrease", fn);
    if (seq_begin[g + 1] > seq_begin[g] && !block_tables[g])
      return fail(PA_ERR_INVALID, "%s: group %d has sequences but no table", fn, g);
  }
  const int32_t num_seqs = seq_begin[num_groups];
  if (num_seqs > 65535) return fail(PA_ERR_INVALID, "%s: num_seqs %d", fn, num_seqs);
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !context_lens) return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID, "%s: q and out must be 16-byte aligned", fn);
  const pa_pool* p0 = &pools[0];
  if (p0->kv_dtype == PA_FP8_E4M3) {
    if (!valid_io_dtype(q_dtype)) return fail(PA_ERR_INVALID, "%s: q_dtype %d", fn, q_dtype);
  } else if (q_dtype != p0->kv_dtype) {
    return fail(PA_ERR_UNSUPPORTED, "%s: q_dtype %d must equal kv_dtype %d", fn, q_dtype,
                p0->kv_dtype);
  }
  if (out_dtype != PA_F32 && out_dtype != q_dtype)
    return fail(PA_ERR_INVALID, "%s: out_dtype must be f32 or q_dtype", fn);
  const WsLayout w = ws_layout_parts(p0, num_seqs, parts);
  if (w.parts > 1) {
    if (!workspace || size_t(w.bytes) > workspace_bytes || !aligned(workspace, 256))
      return fail(PA_ERR_INVALID, "%s: workspace of %lld bytes, 256-byte aligned, is required",
                  fn, (long long)w.bytes);
  }
  char* ws = static_cast<char*>(workspace);
  pa::DecodeMultiArgs m{};
  pa::DecodeArgs& a = m.base;
  a.out = out;
  a.q = q;
  a.context_lens = context_lens;
  a.ws_ml = w.parts > 1 ? reinterpret_cast<float*>(ws + w.ml_off) : nullptr;
  a.ws_acc = w.parts > 1 ? reinterpret_cast<float*>(ws + w.acc_off) : nullptr;
  a.num_heads = p0->num_heads;
  a.max_parts = w.parts < 1 ? 1 : w.parts;
  a.ws_parts = a.max_parts;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.q_dtype = q_dtype;
  a.out_dtype = out_dtype;
  m.num_groups = num_groups;
  m.part_tokens = pt;
  bool stream_v = true;
  for (int32_t g = 0; g < num_groups; ++g) {
    pa::DecodeGroup& d = m.g[g];
    d.k_cache = pools[g].k_cache;
    d.v_cache = pools[g].v_cache;
    d.k_scale = pools[g].k_scale;
    d.v_scale = pools[g].v_scale;
    d.block_tables = block_tables[g];
    d.max_blocks_per_seq = max_blocks_per_seq[g];
    d.block_size = pools[g].block_size;
    d.seq_begin = seq_begin[g];
    stream_v = stream_v && (pools[g].flags & PA_POOL_STREAM_KV) != 0;
  }
  return hip_status(fn, pa::launch_decode_multi(m, p0->kv_dtype, p0->head_dim, stream_v,
                                                num_seqs, stream));
}

pa_status pa_prefill_chunk(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                           const pa_pool* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* query_start_loc, int32_t num_seqs,
                           int32_t max_query_len, float scale, hipStream_t stream) {
  const char* fn = "pa_prefill_chunk";
  if (pa_status s = check_pool(fn, pool)) return s;
  if (num_seqs < 0 || num_seqs > 65535) return fail(PA_ERR_INVALID, "%s: num_seqs %d", fn, num_seqs);
  if (num_seqs == 0 || max_query_len == 0) return PA_OK;
  if (max_query_len < 0) return fail(PA_ERR_INVALID, "%s: max_query_len < 0", fn);
  if (!out || !q || !block_tables || !context_lens || !query_start_loc)
    return fail(PA_ERR_INVALID, "%s: NULL argument", fn);
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(PA_ERR_INVALID, "%s: q and out must be 16-byte aligned", fn);
  if (!row_fits(pool, max_blocks_per_seq))
    return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq %d (1..INT32_MAX / block_size)", fn,
                max_blocks_per_seq);
  if (pool->kv_dtype == PA_FP8_E4M3) {
    if (q_dtype != PA_F16 && q_dtype != PA_BF16)
      return fail(PA_ERR_UNSUPPORTED, "%s: q_dtype %d (fp8 pools: f16 or bf16)", fn, q_dtype);
  } else if (pool->kv_dtype != PA_F16 && pool->kv_dtype != PA_BF16) {
    return fail(PA_ERR_UNSUPPORTED, "%s: kv_dtype %d (built: f16, bf16, fp8)", fn, pool->kv_dtype);
  } else if (q_dtype != pool->kv_dtype) {
    return fail(PA_ERR_UNSUPPORTED, "%s: q_dtype must equal kv_dtype", fn);
  }
  if (out_dtype != PA_F32 && out_dtype != q_dtype)
    return fail(PA_ERR_INVALID, "%s: out_dtype must be f32 or q_dtype", fn);
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = pool->k_cache;
  a.v_cache = pool->v_cache;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = pool->num_heads;
  a.num_seqs = num_seqs;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_dtype = out_dtype;
  return hip_status(fn, pa::launch_prefill(a, pool->kv_dtype, q_dtype, pool->head_dim,
                                           pool->block_size, max_query_len, stream));
}

}  // extern "C"
