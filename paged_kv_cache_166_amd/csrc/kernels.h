// Host-side view of the kernels: argument blocks and launchers (internal to
// libpa.so; the public surface is include/pa.h).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;    // [num_seqs][num_heads][max_parts][head_dim]
  float* ws_ml;     // [num_seqs][num_heads][max_parts][2]  (max, sum)
  int32_t max_blocks_per_seq;
  int32_t num_heads;
  int32_t block_size;
  int32_t part_blocks;
  int32_t max_parts;
  float scale_log2;  // scale * log2(e)
  int32_t q_dtype;
  int32_t out_dtype;
  // pa_decode_append only (else NULL): the new row of each sequence,
  // [num_seqs][num_heads][head_dim] of the KV type (fp8 pools: of q_dtype,
  // quantised on the way in), and its slot (< 0: none)
  const void* k_new;
  const void* v_new;
  const int64_t* new_slots;
  // fp8 pools with PA_POOL_FP8_AUTO_SCALE: the new rows keep each block's
  // scale at amax / 448 (earlier rows requantised when it grows)
  int32_t fp8_upkeep;
  // pa_decode_shared_prefix only (else 0): the first first_block blocks of
  // every table are the shared prefix, attended elsewhere into partitions
  // 0 .. prefix_parts-1; this launch covers the blocks after them, into
  // partitions prefix_parts onwards.
  int32_t first_block;
  int32_t prefix_parts;
  // partitions per (sequence, head) in the workspace (its stride): max_parts,
  // or more when other launches own some of them (prefix_parts)
  int32_t ws_parts;
  // pa_decode_shared_prefix when every sequence's own blocks fit one
  // partition: the workgroup of that partition (of partition 0 when there
  // are none) merges the prefix's partials with its own and writes the
  // output, so no merge launch follows.
  int32_t fuse_merge;
};

hipError_t launch_decode(const DecodeArgs& a, int kv_dtype, int head_dim, int block_size,
                         bool stream_v, int num_seqs, hipStream_t stream);

// One pool of a batch over several pools (pa_decode_multi).
struct DecodeGroup {
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;  // this group's rows only
  int32_t max_blocks_per_seq;
  int32_t block_size;
  int32_t seq_begin;            // first batch row of the group
  int32_t pad;
};

constexpr int kMaxDecodeGroups = 8;

struct DecodeMultiArgs {
  DecodeArgs base;  // q, out, context_lens, workspace, heads, max_parts, scale, dtypes
  int32_t num_groups;
  int32_t part_tokens;
  DecodeGroup g[kMaxDecodeGroups];
};

hipError_t launch_decode_multi(const DecodeMultiArgs& m, int kv_dtype, int head_dim,
                               bool stream_v, int num_seqs, hipStream_t stream);

struct CacheWriteArgs {
  void* k_cache;
  void* v_cache;
  float* k_scale;     // fp8: read, and with scale_upkeep also written
  float* v_scale;
  const void* key;
  const void* value;
  const int64_t* slots;
  int32_t num_tokens;
  int32_t num_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t in_dtype;
  int32_t kv_dtype;
  int32_t scale_upkeep;  // fp8: keep each (block, head) scale at the rows' amax / 448
};

hipError_t launch_reshape_and_cache(const CacheWriteArgs& a, hipStream_t stream);

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  const int32_t* src_dst;
  int32_t num_pairs;
  int32_t num_heads;
  int64_t tile_bytes;  // block_size * head_dim * element size
};

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;  // fp8 pools: [num_blocks][num_heads]
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;
  int32_t max_blocks_per_seq;
  int32_t num_heads;
  int32_t num_seqs;
  float scale_log2;
  int32_t out_dtype;
  // Shared-prefix partials (pa_decode_shared_prefix) only: every query row
  // is one sequence's decode query; keys are the first prefix_len tokens of
  // sequence 0's table, in chunks of chunk_keys; each chunk's (max, sum,
  // unnormalised output) goes to partition `chunk` of the decode workspace.
  float* ws_acc;
  float* ws_ml;
  int32_t max_parts;
  int32_t prefix_len;
  int32_t chunk_keys;
};

hipError_t launch_prefill(const PrefillArgs& a, int kv_dtype, int q_dtype, int head_dim,
                          int block_size, int max_query_len, hipStream_t stream);
hipError_t launch_prefix_partials(const PrefillArgs& a, int kv_dtype, int q_dtype, int head_dim,
                                  int block_size, hipStream_t stream);

// Device address of the fixed split-K scratch of pa_decode_noalloc on the
// GPU of `stream` (looked up once per GPU).
hipError_t noalloc_scratch(hipStream_t stream, void** out);

}  // namespace pa
