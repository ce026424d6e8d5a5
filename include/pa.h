/*
 * pa.h -- C ABI of libpa.so, paged attention for AMD Instinct MI355X (gfx950).
 *
 * The KV cache is split into fixed-size blocks of tokens that sit anywhere in
 * one physical pool; each sequence's block table maps its logical blocks to
 * physical ones and its length truncates the last, partly filled block
 * (vLLM course ch. 4 "PagedAttention core idea"; DataWhale llm-algo-leetcode
 * (5) notes, "vLLM PagedAttention" section 3).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Device pointers are owned by the caller (e.g. torch tensors).  The GPU
 *   calls never allocate, free or synchronise device memory; every launch goes
 *   on the caller's stream and returns before the GPU work ends.
 * - Every call returns pa_status.  0 is success, negative is an error; nothing
 *   is launched when an argument check fails.  pa_last_error() returns a
 *   message for the last failing call of the calling thread.  Faults inside a
 *   kernel surface at the caller's next synchronisation of the stream.
 * - Host-side checks: null pointers, dtype combinations, head_dim in {64,128},
 *   block_size in {4,8,16,32,64}, 16-byte alignment of every device pointer,
 *   workspace size, and table rows of 1..INT32_MAX / block_size entries
 *   (max_blocks_per_seq; lengths are int32, so no row can address more).
 *   Block-table entries and slots are trusted: the caller keeps them in
 *   [0, num_blocks) (the allocator below produces only such).
 * - Pool layout: K and V are each [num_blocks][num_heads][block_size][head_dim]
 *   of kv_dtype, so one (block, head) tile is contiguous (block_size*head_dim
 *   elements; 4 KiB for 16 x 128 fp16).  Pool bases must be 128-byte aligned,
 *   the alignment the course ch. 4 pitfall note asks for.
 * - fp8 pools (PA_FP8_E4M3, OCP E4M3FN, max 448) carry one float32 scale per
 *   (block, head) for K and one for V: value = code * scale (the blog
 *   article's mixed-precision KV storage, section 2.3).
 * - The host allocator is an opaque handle; it is not thread safe; on error
 *   it changes no state.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* bad argument; nothing launched, no state changed */
  PA_ERR_OOM = -2,         /* the free list cannot satisfy the request */
  PA_ERR_UNSUPPORTED = -3, /* valid but not built (dtype / shape combination) */
  PA_ERR_HIP = -4,         /* the HIP runtime reported an error on launch */
  PA_ERR_NO_SEQ = -5       /* unknown sequence id */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3 /* OCP E4M3FN */
} pa_dtype;

/* One layer's paged pool.  All pointers are device pointers. */
typedef struct pa_pool {
  void* k_cache;      /* [num_blocks][num_heads][block_size][head_dim] kv_dtype */
  void* v_cache;      /* same shape as k_cache */
  float* k_scale;     /* [num_blocks][num_heads], fp8 pools only, else NULL */
  float* v_scale;     /* [num_blocks][num_heads], fp8 pools only, else NULL */
  int32_t num_blocks;
  int32_t num_heads;
  int32_t block_size; /* tokens per block: 4, 8, 16, 32 or 64 */
  int32_t head_dim;   /* 64 or 128 */
  int32_t kv_dtype;   /* pa_dtype */
  int32_t flags;      /* PA_POOL_* bits, 0 for none */
} pa_pool;

/*
 * pa_pool.flags
 * PA_POOL_STREAM_KV: no block of the pool is read by more than one sequence
 *   of a pa_decode batch (no prefix sharing or forks in flight), so decode
 *   reads every K/V tile exactly once.  pa_decode then loads V with
 *   non-temporal loads: they skip the cache fills that a read-once stream
 *   does not need (at the LLaMA-13B decode shape about 6% more KV bandwidth).
 *   Leave it clear when blocks are shared: their repeated reads then hit the
 *   caches.  Results are bit-identical either way; other calls ignore it.
 */
#define PA_POOL_STREAM_KV 1

/*
 * PA_POOL_FP8_AUTO_SCALE (fp8 pools only): pa_reshape_and_cache keeps each
 *   (block, head) scale at amax / 448 of the rows the block holds (the blog
 *   article's mixed-precision KV, section 2.3, for blocks that fill a few
 *   tokens at a time), for K and V separately.  The call's tokens are taken
 *   in runs: consecutive tokens whose slots are consecutive positions of one
 *   block.  For each run and head, in float32: s_run = amax(|rows|) / 448;
 *   s_old = 0 if the run starts the block (position 0), else the block's
 *   scale; s_new = max(s_old, s_run).  If s_new > s_old, the block's earlier
 *   rows are requantised, code = RNE-saturate((decode(code) * s_old) /
 *   s_new); the run's rows are stored as RNE-saturate(x / s_new); the scale
 *   becomes s_new.  While a scale is 0 (all values so far zero) the divisor
 *   is 1.  Precondition (what the allocator's slot mappings give): each
 *   block's new rows form one run of the call, after the rows the block
 *   already holds.  Without the flag the caller owns the scales and rows are
 *   stored with the block's existing scale.
 */
#define PA_POOL_FP8_AUTO_SCALE 2

/* ---------------------------------------------------------------- GPU calls */

/*
 * pa_reshape_and_cache -- write new K/V rows into their pool slots.
 * Slot s is block s / block_size, row s % block_size (vLLM course ch. 4,
 * attention pseudocode: the block table gives the physical block, the row
 * inside it is the token's offset).
 *   key, value    device, [num_tokens][num_heads][head_dim] of in_dtype,
 *                 contiguous.  For f32/f16/bf16 pools in_dtype must equal
 *                 kv_dtype and the rows are copied bit for bit.  For fp8 pools
 *                 in_dtype is f32, f16 or bf16 and each element is stored as
 *                 RNE-saturate(x / scale[block][head]) with the division in
 *                 float32; the block's scale must already be set, unless the
 *                 pool has PA_POOL_FP8_AUTO_SCALE (then the call maintains
 *                 the scales, see that flag).
 *   slot_mapping  device, [num_tokens] int64; a negative slot skips the row.
 * Two rows of one call must not name the same slot.
 */
pa_status pa_reshape_and_cache(const pa_pool* pool, const void* key, const void* value,
                               int32_t in_dtype, const int64_t* slot_mapping,
                               int32_t num_tokens, hipStream_t stream);

/*
 * pa_copy_blocks -- whole-block copy of K and V (and of the fp8 scales) for
 * each (src, dst) pair, the copy that copy-on-write needs before a sequence
 * writes into a block it shares (DataWhale notes section 4, copy-on-write).
 *   src_dst   device, [num_pairs][2] int32.  Pairs are independent: no dst may
 *             be another pair's src or dst.
 */
pa_status pa_copy_blocks(const pa_pool* pool, const int32_t* src_dst, int32_t num_pairs,
                         hipStream_t stream);

/*
 * Partition size chosen by pa_decode when partition_blocks == 0, for this
 * pool and batch.  Exposed so that callers can size the workspace.
 */
int32_t pa_decode_auto_partition_blocks(const pa_pool* pool, int32_t num_seqs,
                                        int32_t max_blocks_per_seq);

/*
 * Bytes of device workspace pa_decode needs for these arguments (0 when every
 * sequence fits in one partition, and for arguments pa_decode would refuse):
 * the (max, sum) pair and the unnormalised output of every (sequence, head,
 * partition), float32.  No initialisation is needed.
 */
size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, int32_t partition_blocks);

/*
 * pa_decode -- attention of one query token per sequence over its paged K/V
 * (blog article section 3.2.2 forward pass at one query row; vLLM course
 * ch. 4 attention pseudocode).  For sequence i and head h, with L = context
 * length (every cached token, the current one included):
 *     out[i][h] = sum_j softmax_j(scale * <q[i][h], K_i[j][h]>) V_i[j][h],
 * j over 0..L-1 gathered through the block table; L = 0 gives zeros.
 *   out           device, [num_seqs][num_heads][head_dim] of out_dtype
 *                 (f32, or q_dtype).
 *   q             device, [num_seqs][num_heads][head_dim] of q_dtype
 *                 (kv_dtype for f32/f16/bf16 pools; f32/f16/bf16 for fp8).
 *   block_tables  device, [num_seqs][max_blocks_per_seq] int32; only the first
 *                 ceil(L / block_size) entries of a row are read.
 *   context_lens  device, [num_seqs] int32, 0 <= L <= max_blocks_per_seq*block_size.
 *   partition_blocks  blocks per split-K partition, 1..256 (0 = automatic).
 *                 Sequences longer than one partition are split; the
 *                 partitions' (max, sum, output) triples are merged by a
 *                 second, small kernel on the same stream.  At most 65535
 *                 partitions per sequence (ceil(max_blocks_per_seq /
 *                 partition_blocks)); more is PA_ERR_UNSUPPORTED.
 *   workspace     device, >= pa_decode_workspace_bytes(...) bytes, 256-byte
 *                 aligned (may be NULL when that is 0).  Calls that share a
 *                 workspace must be ordered (same stream).
 */
pa_status pa_decode(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                    const pa_pool* pool, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    float scale, int32_t partition_blocks, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results as pa_decode
 * (bit for bit), without the workspace: the split-K scratch is a fixed
 * array of PA_DECODE_NOALLOC_MAX_WORKSPACE bytes in device memory, one per
 * GPU, held by every GPU the library runs on until the process ends.  Its
 * address on a GPU is looked up on the first call that runs there (on the
 * device of `stream`); no call allocates or frees anything.
 *   A batch whose split-K needs more than that
 *   (pa_decode_workspace_bytes(...) > PA_DECODE_NOALLOC_MAX_WORKSPACE) is
 *   PA_ERR_UNSUPPORTED, before any launch; use pa_decode with a workspace.
 *   Calls on one GPU share the array: two that overlap in time (different
 *   streams with no ordering between them) race on it and give undefined
 *   results.  Calls on one stream, or otherwise ordered, are safe; nothing
 *   in the array needs clearing between calls.
 */
#define PA_DECODE_NOALLOC_MAX_WORKSPACE (32u << 20)
pa_status pa_decode_noalloc(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                            const pa_pool* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, float scale, int32_t partition_blocks,
                            hipStream_t stream);

/*
 * pa_decode_append -- pa_reshape_and_cache of each sequence's new token,
 * then pa_decode, in one launch (same results, same cache contents).  The
 * new row belongs to position context_lens[i] - 1 of sequence i: the
 * workgroup that covers that position stores the row at new_slots[i] and
 * uses it from registers, so the row is never read back in this call.
 *   key_new, value_new  device, [num_seqs][num_heads][head_dim] of q_dtype
 *                 (which is the pool's type for f32, f16 and bf16 pools),
 *                 16-byte aligned.  fp8 pools quantise them on the way in as
 *                 pa_reshape_and_cache does: with PA_POOL_FP8_AUTO_SCALE the
 *                 block's scale is kept up (its earlier rows requantised in
 *                 the launch when it grows, and attended as requantised),
 *                 else the block's scale is used as it is.
 *   new_slots     device, [num_seqs] int64: the slot of position
 *                 context_lens[i] - 1 (what pa_append_tokens returned);
 *                 < 0: no row for that sequence (nothing stored, the cache is
 *                 read as it is).  The slot's block must not be shared (copy it
 *                 first, as for any write).
 * Other arguments, layout and errors as pa_decode.
 */
pa_status pa_decode_append(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                           const pa_pool* pool, const void* key_new, const void* value_new,
                           const int64_t* new_slots, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, float scale, int32_t partition_blocks,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_shared_prefix -- pa_decode of a batch whose sequences all begin
 * with the same physical blocks (prefix sharing by copy-on-write, the
 * DataWhale notes' section 4): the shared prefix is read once for the whole
 * batch instead of once per sequence.  Same result as pa_decode up to the
 * order of the floating-point sums (the same tolerance applies).
 *   1. every sequence's query against the prefix keys, as a multi-query
 *      pass on MFMA (the prefill kernel's tiles, no mask), chunk by chunk,
 *      each chunk's (max, sum, unnormalised output) into the workspace;
 *   2. each sequence's own blocks after the prefix, split into partitions of
 *      partition_blocks (0: automatic) as in pa_decode, into the workspace;
 *   3. the merge of all of them: by the workgroup of step 2 when every
 *      sequence's own blocks fit one partition (max_blocks_per_seq -
 *      shared_blocks <= the partition size), else by a third launch.
 *   shared_blocks  the first shared_blocks entries of every row of
 *                 block_tables are the same blocks, and every sequence's
 *                 context covers them (context_lens[i] >= shared_blocks *
 *                 block_size); 1 <= shared_blocks <= max_blocks_per_seq.  Not
 *                 checked on the device.
 * f16, bf16 and fp8 pools (PA_ERR_UNSUPPORTED for f32); q of the pool's
 * type, or f16 / bf16 for fp8 pools (the prefix pass runs on MFMA).  Value
 * range: the prefix pass has pa_prefill_chunk's bound on V (bf16 pools:
 * |v| <= 65504, see there), which pa_decode does not have.  A
 * workspace is always needed:
 * pa_decode_shared_prefix_workspace_bytes(...).  Other arguments as pa_decode.
 */
size_t pa_decode_shared_prefix_workspace_bytes(const pa_pool* pool, int32_t num_seqs,
                                               int32_t max_blocks_per_seq, int32_t shared_blocks,
                                               int32_t partition_blocks);
pa_status pa_decode_shared_prefix(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                  const pa_pool* pool, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t shared_blocks, float scale,
                                  int32_t partition_blocks, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_shared_prefix_append -- pa_decode_shared_prefix with the step's
 * new K/V row of each sequence stored and attended in the same launch, as
 * pa_decode_append does for pa_decode (same results and cache contents as
 * pa_reshape_and_cache of those rows followed by pa_decode_shared_prefix).
 *   key_new, value_new, new_slots  as in pa_decode_append; the new row's
 *                 position context_lens[i] - 1 lies past the shared blocks
 *                 (a row is never written into a shared block).
 * Other arguments, workspace and errors as pa_decode_shared_prefix (f16, bf16
 * and fp8 pools, the new rows of fp8 pools quantised as in pa_decode_append).
 */
pa_status pa_decode_shared_prefix_append(void* out, int32_t out_dtype, const void* q,
                                         int32_t q_dtype, const pa_pool* pool,
                                         const void* key_new, const void* value_new,
                                         const int64_t* new_slots, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t shared_blocks, float scale,
                                         int32_t partition_blocks, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_multi -- pa_decode of one batch whose sequences live in several
 * pools with the same num_heads, head_dim and kv_dtype (typically the
 * block-size views of one arena, pa_buddy_*), in one launch (plus the merge
 * launch when a sequence spans more than one partition).  Rows of out, q and
 * context_lens are grouped by pool: group g is rows [seq_begin[g],
 * seq_begin[g+1]) and uses pools[g] and block_tables[g].
 *   pools           host, [num_groups] (1..8).
 *   block_tables    host array of num_groups device pointers; group g's
 *                   tables are [rows of g][max_blocks_per_seq[g]] int32 in
 *                   pools[g]'s block ids (may be NULL for an empty group).
 *   max_blocks_per_seq  host, [num_groups], each >= 1.
 *   seq_begin       host, [num_groups + 1], non-decreasing, seq_begin[0] = 0;
 *                   seq_begin[num_groups] is the batch size.
 *   partition_tokens  tokens per split-K partition in every group (0: 512);
 *                   a multiple of every group's block size, at most 256
 *                   blocks of each.
 *   workspace       >= pa_decode_multi_workspace_bytes(...) bytes.
 * The V loads stream past the caches only if every pool has
 * PA_POOL_STREAM_KV.  Other arguments and errors as pa_decode.
 */
size_t pa_decode_multi_workspace_bytes(const pa_pool* pools, const int32_t* max_blocks_per_seq,
                                       int32_t num_groups, int32_t num_seqs,
                                       int32_t partition_tokens);
pa_status pa_decode_multi(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                          const pa_pool* pools, int32_t num_groups,
                          const int32_t* const* block_tables, const int32_t* max_blocks_per_seq,
                          const int32_t* seq_begin, const int32_t* context_lens, float scale,
                          int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * pa_prefill_chunk -- causal attention of a chunk of query tokens against the
 * sequence's paged context (blog article section 3.2.2 forward pass with its
 * causal mask; the mask is aligned so that the chunk's rows are the last
 * S_i positions of a sequence of L_i tokens: row r sees keys 0 .. L_i - S_i + r).
 * The chunk's own K/V must already be in the pool.
 *   q, out            device, packed [total_q][num_heads][head_dim]; sequence
 *                     i owns rows query_start_loc[i] .. query_start_loc[i+1]-1.
 *                     q_dtype = kv_dtype for f16 and bf16 pools; f16 or bf16
 *                     for fp8 pools (codes times the pool's per-(block, head)
 *                     scales, as in pa_decode; |v| * 2^8 must stay within the
 *                     fp16 range, |v| <= 255 * 448 * scale).  out_dtype f32 or
 *                     q_dtype.
 *                     Value range of V: the P V product runs on fp16 inputs,
 *                     so bf16 pools convert V to fp16 (RNE; exact for every
 *                     bf16 value from 2^-14 to 65280).  Every |v| must be at
 *                     most 65504: a larger value becomes inf, and that
 *                     (head, dimension) of the output turns inf or NaN for
 *                     every row that sees its key (and may for rows of the
 *                     same key tile that do not).  Values below 2^-14 keep
 *                     fp16's subnormal spacing (an absolute error of at most
 *                     2^-25 per value).  Not checked.
 *   query_start_loc   device, [num_seqs + 1] int32, non-decreasing, from 0.
 *   context_lens      device, [num_seqs] int32, S_i <= L_i <=
 *                     max_blocks_per_seq * block_size (chunk included); the
 *                     first ceil(L_i / block_size) table entries are read.
 *   max_query_len     host bound on every S_i (sizes the grid).
 */
pa_status pa_prefill_chunk(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                           const pa_pool* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* query_start_loc, int32_t num_seqs,
                           int32_t max_query_len, float scale, hipStream_t stream);

/* ------------------------------------------------------ host block allocator */

/*
 * The block manager of the pages: a free list of physical blocks, one block
 * table per sequence, ceil(n / block_size) blocks for a prompt, one more block
 * when a decode step crosses a block boundary, "OOM" when the free list runs
 * short, blocks returned when a sequence ends (DataWhale notes, KVCacheManager
 * exercise; vLLM course ch. 4 "Block management strategy" table and allocation
 * flow), and copy-on-write sharing of prefix blocks (DataWhale notes section 4).
 * The free list is FIFO: blocks are taken from its front, freed blocks go to
 * its back in table order.  All pointers here are host pointers.
 */
typedef struct pa_allocator pa_allocator;

/* initial_free_order: [num_blocks] permutation of 0..num_blocks-1, or NULL for
 * 0, 1, ..., num_blocks-1. */
pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* initial_free_order, pa_allocator** out);
void pa_allocator_destroy(pa_allocator* a);

/* New sequence of num_tokens tokens (ceil(num_tokens / block_size) blocks,
 * all or nothing).  slots_out: [num_tokens] or NULL. */
pa_status pa_alloc_prompt(pa_allocator* a, int64_t seq_id, int32_t num_tokens,
                          int64_t* slots_out);

/* Append n tokens.  If the last block is partly filled and shared, one fresh
 * block is taken first and (src, dst) is returned for a whole-block copy
 * (cow_src_dst[2], *num_cow = 1; else *num_cow = 0); then
 * ceil((L+n)/bs) - ceil(L/bs) new blocks.  slots_out: [n] or NULL.
 * A sequence holds at most INT32_MAX tokens (lengths leave the allocator as
 * int32): an append past that is PA_ERR_INVALID, here and in the batch call. */
pa_status pa_append_tokens(pa_allocator* a, int64_t seq_id, int32_t n, int64_t* slots_out,
                           int32_t* cow_src_dst, int32_t* num_cow);

/* Append n tokens to each of num_seqs distinct sequences, all or nothing
 * (the whole batch is checked against the free list first).  slots_out:
 * [num_seqs][n]; cow_pairs_out: [num_seqs][2] (a sequence's pair, or -1 -1);
 * *num_cow: number of copies. */
pa_status pa_append_tokens_batch(pa_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                                 int32_t n, int64_t* slots_out, int32_t* cow_pairs_out,
                                 int32_t* num_cow);

/* The child shares every block of the parent (reference count + 1). */
pa_status pa_fork(pa_allocator* a, int64_t parent_id, int64_t child_id);

/* Drop the sequence; blocks whose reference count reaches 0 return to the back
 * of the free list in table order. */
pa_status pa_free_seq(pa_allocator* a, int64_t seq_id);

/* Copy a block table out: up to cap entries into out, *len = table length,
 * *seq_len = tokens (either output may be NULL). */
pa_status pa_get_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                             int32_t* len, int32_t* seq_len);

/* Padded tables for a batch: tables_out [num_seqs][max_blocks] (-1 padding),
 * lens_out [num_seqs] (either may be NULL). */
pa_status pa_pack_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                               int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

int32_t pa_num_free_blocks(const pa_allocator* a);
int32_t pa_block_refcount(const pa_allocator* a, int32_t block);

/* Counters: [0] blocks in use, [1] blocks shared (refcount > 1), [2] copies
 * made by copy-on-write, [3] OOM refusals, [4] live sequences. */
pa_status pa_allocator_stats(const pa_allocator* a, int64_t* out5);

/* ------------------------------------------------------- host prefix index */

/*
 * A prefix index over token ids bound to one allocator (the DataWhale notes'
 * RadixAttention section: cached token sequences in a radix tree whose
 * nodes point at the physical KV blocks; a new prompt reuses the blocks of
 * its longest cached prefix and only the rest is computed; an edge is split
 * where a new sequence leaves it).  Token ids are int32.  Not thread-safe;
 * destroy the index before its allocator.  A host allocation failure inside
 * an index call (PA_ERR_OOM with a "host allocation failed" message, as
 * opposed to the allocator's block OOM, which changes nothing) may leave the
 * index part-way through that call: clear it (pa_prefix_clear) before
 * using it again.
 *
 * Blocks: an inserted sequence is an entry.  It provides the positions from
 * its divergence point d (its match length before insertion) to its end and
 * holds one allocator reference on each of its blocks covering one of them
 * (indices d / bs .. (n-1) / bs), so cached blocks outlive the sequence.
 * Block j of a hit of h tokens is block j of the earliest entry whose common
 * prefix with the prompt is longer than min((j+1) * bs, h) - 1.
 *
 * Eviction (the same section's LRU rule for a full memory: leaves of the
 * tree go first, least recently used first, until there is room).  Every
 * pa_prefix_insert and pa_alloc_prompt_cached stamps the tree nodes its walk
 * entered with a logical clock (pa_prefix_match stamps nothing); the oldest
 * leaf goes first, ties to the older node.  Evicting a leaf drops its
 * creating entry's references on the blocks only that leaf uses (the block
 * under its first position stays when the parent node, made by the same
 * entry, also lies in it); a block left with no reference goes back to the
 * free list.  Blocks of live sequences are never taken.
 */
typedef struct pa_prefix_index pa_prefix_index;

pa_status pa_prefix_index_create(pa_allocator* a, pa_prefix_index** out);
/* Releases the index's references (as pa_prefix_clear), then frees it. */
void pa_prefix_index_destroy(pa_prefix_index* x);

/* Cache the first num_tokens tokens of live sequence seq_id (which holds at
 * least that many).  *divergence (may be NULL) receives d.  A sequence that
 * later writes into a partly filled block the index references copies it
 * first (copy-on-write). */
pa_status pa_prefix_insert(pa_prefix_index* x, int64_t seq_id, const int32_t* tokens,
                           int32_t num_tokens, int32_t* divergence);

/* Longest common prefix of tokens with any cached entry. */
pa_status pa_prefix_match(const pa_prefix_index* x, const int32_t* tokens, int32_t num_tokens,
                          int32_t* hit_len);

/* New sequence seq_id for a prompt of num_tokens tokens: the blocks of its
 * longest cached prefix (h tokens, one reference each), length h, then an
 * append of the other num_tokens - h tokens: slots_out[0 .. num_tokens-h)
 * receives their slots, and (*cow_src_dst, *num_cow = 1) the whole-block
 * copy needed when the hit ends inside a block.  All or nothing: OOM
 * changes nothing.  A full hit leaves no suffix. */
pa_status pa_alloc_prompt_cached(pa_prefix_index* x, int64_t seq_id, const int32_t* tokens,
                                 int32_t num_tokens, int32_t* hit_len, int64_t* slots_out,
                                 int32_t* cow_src_dst, int32_t* num_cow);

/* Drop every entry: references released entry by entry in insertion order,
 * each entry's blocks by index (blocks reaching zero go back to the free
 * list in that order). */
pa_status pa_prefix_clear(pa_prefix_index* x);

/* [0] entries inserted since creation or the last clear, [1] live tree nodes
 * (root included), [2] block references held, [3] leaves evicted so far,
 * [4] node slots in memory (live nodes plus evicted ones not yet dropped:
 * evicted nodes and the entries nothing uses any more are dropped once they
 * outnumber the live nodes by more than 64, so memory stays proportional to
 * what is cached). */
pa_status pa_prefix_stats(const pa_prefix_index* x, int64_t* out5);

/* Switch automatic eviction on (enable != 0) or off for x.  While on, an
 * allocating call on x's allocator (pa_alloc_prompt, pa_append_tokens,
 * pa_append_tokens_batch, pa_alloc_prompt_cached) that would run out of
 * blocks first evicts leaves of x until its demand fits, re-evaluating the
 * demand after every eviction (a block that loses the index's reference may
 * need no copy any more); pa_alloc_prompt_cached never evicts the nodes of
 * its own hit.  If evicting every other leaf would not be enough, the
 * evictions are undone and the call fails with PA_ERR_OOM, nothing changed.
 * One evicting index per allocator: PA_ERR_INVALID if another has it on.
 * Off by default (the allocator then reports OOM when its free list is
 * short). */
pa_status pa_prefix_set_auto_evict(pa_prefix_index* x, int32_t enable);

/* Evict oldest leaves until the allocator has min_free_blocks free blocks
 * or no leaf is left; *num_evicted (may be NULL) receives the count. */
pa_status pa_prefix_evict(pa_prefix_index* x, int64_t min_free_blocks, int64_t* num_evicted);

/* ------------------------------------- host allocator, block size per request */

/*
 * One arena per layer shared by blocks of 8, 16, 32 and 64 tokens, the block
 * size following the request's length (the first page's "3.0" feature list:
 * page size adjusted to the request, blocks of different sizes for requests
 * of different lengths).  The arena is a binary buddy system of 8-token
 * units: a block of b tokens is b/8 units starting at a multiple of b/8.
 * Pool views: for each b the same K and V memory is a pa_pool of block_size
 * b and num_blocks arena_tokens / b, and block id i of that view is units
 * [i*b/8, (i+1)*b/8).  A sequence's table holds block ids of the view of its
 * own size, so pa_reshape_and_cache, pa_copy_blocks, pa_decode and
 * pa_prefill_chunk run on that view unchanged (a batch mixing sizes is one
 * call per size).  fp8 arenas need one scale array per view ([arena_tokens /
 * b][heads]); a block's scales live in the array of its view.
 *
 * Size rule (pa_buddy_size_for): the largest b with b <= n / 16, at least 8:
 * a request starts with 16 or more blocks, so its unfilled tail is under
 * 1/16 of it.  A sequence keeps its size for life.
 *
 * Free lists: one FIFO per size; the arena starts as its 64-token blocks in
 * top_order (NULL: ascending).  A request for size b takes the front of the
 * b list, else splits the front of the nearest larger non-empty list,
 * keeping the lower half and putting each upper half at the back of the list
 * below; a freed block merges with its buddy while the buddy is free at the
 * same size, then goes to the back of its list.  Reference counts, fork,
 * copy-on-write and the all-or-nothing rule are those of pa_allocator; slots
 * are block_id * b + offset in the sequence's view.  Not thread-safe.
 */
typedef struct pa_buddy_allocator pa_buddy_allocator;

/* arena_tokens: a positive multiple of 64. */
pa_status pa_buddy_create(int64_t arena_tokens, const int32_t* top_order, pa_buddy_allocator** out);
void pa_buddy_destroy(pa_buddy_allocator* a);
/* The size rule: block size for a request of num_tokens tokens. */
int32_t pa_buddy_size_for(int64_t num_tokens);
/* New sequence of num_tokens tokens in blocks of block_size (0: the size
 * rule); *block_size_out (may be NULL) receives the size, slots_out (may be
 * NULL) num_tokens slots in that size's view. */
pa_status pa_buddy_alloc_prompt(pa_buddy_allocator* a, int64_t seq_id, int32_t num_tokens,
                                int32_t block_size, int32_t* block_size_out, int64_t* slots_out);
/* As pa_append_tokens (the INT32_MAX-token limit included), in the
 * sequence's view. */
pa_status pa_buddy_append_tokens(pa_buddy_allocator* a, int64_t seq_id, int32_t n,
                                 int64_t* slots_out, int32_t* cow_src_dst, int32_t* num_cow);
/* As pa_append_tokens_batch (sequences of any sizes; each row of slots_out
 * and each pair in its own sequence's view). */
pa_status pa_buddy_append_tokens_batch(pa_buddy_allocator* a, const int64_t* seq_ids,
                                       int32_t num_seqs, int32_t n, int64_t* slots_out,
                                       int32_t* cow_pairs_out, int32_t* num_cow);
pa_status pa_buddy_fork(pa_buddy_allocator* a, int64_t parent_id, int64_t child_id);
pa_status pa_buddy_free_seq(pa_buddy_allocator* a, int64_t seq_id);
/* As pa_get_block_table; *block_size (may be NULL) receives the sequence's size. */
pa_status pa_buddy_get_block_table(const pa_buddy_allocator* a, int64_t seq_id, int32_t* out,
                                   int32_t cap, int32_t* len, int32_t* seq_len,
                                   int32_t* block_size);
/* As pa_pack_block_tables; every listed sequence must have the same size
 * (else PA_ERR_INVALID). */
pa_status pa_buddy_pack_block_tables(const pa_buddy_allocator* a, const int64_t* seq_ids,
                                     int32_t num_seqs, int32_t max_blocks, int32_t* tables_out,
                                     int32_t* lens_out);
/* Free tokens (sum over the free lists). */
int64_t pa_buddy_free_tokens(const pa_buddy_allocator* a);
/* The free list of one size, front first, as block ids of that size's view
 * (up to cap of them in out; *len receives the full length). */
pa_status pa_buddy_free_list(const pa_buddy_allocator* a, int32_t block_size, int32_t* out,
                             int32_t cap, int32_t* len);
/* Reference count of block block_id of the block_size view (-1 if out of range). */
int32_t pa_buddy_block_refcount(const pa_buddy_allocator* a, int32_t block_size, int32_t block_id);

const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
