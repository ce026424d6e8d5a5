// Host block allocator behind the pa_allocator_* / pa_alloc_* calls of pa.h.
//
// The block manager the pages describe (DataWhale llm-algo-leetcode (5) notes,
// "vLLM PagedAttention", KVCacheManager exercise; vLLM course ch. 4 "Block
// management strategy" table and allocation flow; copy-on-write from the
// notes' section 4), built for a serving loop:
//
//  * the free list is a fixed-capacity ring (FIFO): take from the front, give
//    back to the back, no allocation after creation;
//  * one reference count per physical block, so forked sequences share blocks
//    and a write into a shared, partly filled last block copies it first;
//  * every operation validates and counts its whole demand before touching any
//    state, so an error (including OOM) leaves the allocator unchanged;
//  * a batch append for the decode step of many sequences, so one call does
//    the per-step host work of a whole batch.
#include <climits>
#include <algorithm>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "status.h"

#include "allocator_impl.h"

using pa_alloc::blocks_for;
using pa_alloc::Sequence;

extern "C" {

pa_status pa_allocator_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* initial_free_order, pa_allocator** out) {
  if (!out) return pa::fail(PA_ERR_INVALID, "pa_allocator_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pa::fail(PA_ERR_INVALID, "pa_allocator_create: num_blocks=%d block_size=%d",
                    num_blocks, block_size);
  pa_allocator* a = new (std::nothrow) pa_allocator();
  if (!a) return pa::fail(PA_ERR_OOM, "pa_allocator_create: host allocation failed");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ring.resize(num_blocks);
  a->refs.assign(num_blocks, 0);
  if (initial_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = initial_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return pa::fail(PA_ERR_INVALID,
                        "pa_allocator_create: initial_free_order is not a permutation");
      }
      seen[b] = 1;
      a->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->ring[i] = i;
  }
  a->count = num_blocks;
  *out = a;
  return PA_OK;
}

void pa_allocator_destroy(pa_allocator* a) { delete a; }

pa_status pa_alloc_prompt(pa_allocator* a, int64_t seq_id, int32_t num_tokens,
                          int64_t* slots_out) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_alloc_prompt: allocator is NULL");
  if (num_tokens < 0) return pa::fail(PA_ERR_INVALID, "pa_alloc_prompt: num_tokens < 0");
  if (a->seqs.count(seq_id))
    return pa::fail(PA_ERR_INVALID, "pa_alloc_prompt: sequence %lld exists", (long long)seq_id);
  int64_t need = blocks_for(num_tokens, a->block_size);
  if (a->short_of([&] { return need; })) {
    ++a->oom_refusals;
    return pa::fail(PA_ERR_OOM, "OOM: prompt needs %lld blocks, %lld free", (long long)need,
                    (long long)a->count);
  }
  Sequence& s = a->seqs[seq_id];
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(a->take());
  s.len = num_tokens;
  if (slots_out)
    for (int64_t p = 0; p < num_tokens; ++p) slots_out[p] = a->slot(s, p);
  return PA_OK;
}

pa_status pa_append_tokens(pa_allocator* a, int64_t seq_id, int32_t n, int64_t* slots_out,
                           int32_t* cow_src_dst, int32_t* num_cow) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_append_tokens: allocator is NULL");
  if (n < 0) return pa::fail(PA_ERR_INVALID, "pa_append_tokens: n < 0");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_append_tokens: no sequence %lld", (long long)seq_id);
  Sequence& s = it->second;
  if (s.len + n > INT32_MAX)   // lengths leave the allocator as int32
    return pa::fail(PA_ERR_INVALID, "pa_append_tokens: sequence %lld would pass INT32_MAX tokens",
                    (long long)seq_id);
  auto need_now = [&] {
    bool cow = false;
    return a->demand(s, n, s.table.empty() ? 0 : a->refs[s.table.back()], &cow);
  };
  if (a->short_of(need_now)) {
    const int64_t need = need_now();
    ++a->oom_refusals;
    return pa::fail(PA_ERR_OOM, "OOM: append needs %lld blocks, %lld free", (long long)need,
                    (long long)a->count);
  }
  int32_t pair[2];
  a->apply_append(s, n, slots_out, pair);
  if (cow_src_dst) {
    cow_src_dst[0] = pair[0];
    cow_src_dst[1] = pair[1];
  }
  if (num_cow) *num_cow = pair[0] >= 0 ? 1 : 0;
  return PA_OK;
}

pa_status pa_append_tokens_batch(pa_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                                 int32_t n, int64_t* slots_out, int32_t* cow_pairs_out,
                                 int32_t* num_cow) {
  if (!a || (!seq_ids && num_seqs > 0))
    return pa::fail(PA_ERR_INVALID, "pa_append_tokens_batch: NULL argument");
  if (n < 0 || num_seqs < 0) return pa::fail(PA_ERR_INVALID, "pa_append_tokens_batch: negative size");
  std::unordered_set<int64_t> ids;
  std::vector<const Sequence*> listed(num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (!ids.insert(seq_ids[i]).second)
      return pa::fail(PA_ERR_INVALID, "pa_append_tokens_batch: sequence %lld listed twice",
                      (long long)seq_ids[i]);
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return pa::fail(PA_ERR_NO_SEQ, "pa_append_tokens_batch: no sequence %lld",
                      (long long)seq_ids[i]);
    if (it->second.len + n > INT32_MAX)
      return pa::fail(PA_ERR_INVALID,
                      "pa_append_tokens_batch: sequence %lld would pass INT32_MAX tokens",
                      (long long)seq_ids[i]);
    listed[i] = &it->second;
  }
  // Dry run: the reference counts the batch's own copies leave behind decide
  // whether a later sequence of the batch still shares its last block.
  std::unordered_map<int32_t, int32_t> dropped;
  auto need_now = [&] {
    dropped.clear();
    int64_t need = 0;
    for (const Sequence* s : listed) {
      int32_t last = s->table.empty() ? -1 : s->table.back();
      int32_t last_refs = last < 0 ? 0 : a->refs[last] - (dropped.count(last) ? dropped[last] : 0);
      bool cow = false;
      need += a->demand(*s, n, last_refs, &cow);
      if (cow) ++dropped[last];
    }
    return need;
  };
  if (a->short_of(need_now)) {
    const int64_t need = need_now();
    ++a->oom_refusals;
    return pa::fail(PA_ERR_OOM, "OOM: batch append needs %lld blocks, %lld free",
                    (long long)need, (long long)a->count);
  }
  int32_t copies = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Sequence& s = a->seqs[seq_ids[i]];
    int32_t pair[2];
    a->apply_append(s, n, slots_out ? slots_out + int64_t(i) * n : nullptr, pair);
    if (cow_pairs_out) {
      cow_pairs_out[2 * i] = pair[0];
      cow_pairs_out[2 * i + 1] = pair[1];
    }
    if (pair[0] >= 0) ++copies;
  }
  if (num_cow) *num_cow = copies;
  return PA_OK;
}

pa_status pa_fork(pa_allocator* a, int64_t parent_id, int64_t child_id) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_fork: allocator is NULL");
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_fork: no sequence %lld", (long long)parent_id);
  if (a->seqs.count(child_id))
    return pa::fail(PA_ERR_INVALID, "pa_fork: sequence %lld exists", (long long)child_id);
  Sequence child = it->second;  // copy before inserting (rehash safety)
  for (int32_t b : child.table) ++a->refs[b];
  a->seqs.emplace(child_id, std::move(child));
  return PA_OK;
}

pa_status pa_free_seq(pa_allocator* a, int64_t seq_id) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_free_seq: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_free_seq: no sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.table)
    if (--a->refs[b] == 0) a->give_back(b);
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_get_block_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t cap,
                             int32_t* len, int32_t* seq_len) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_get_block_table: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_get_block_table: no sequence %lld", (long long)seq_id);
  const Sequence& s = it->second;
  int32_t n = int32_t(s.table.size());
  if (out) std::copy_n(s.table.begin(), std::min(n, std::max(cap, 0)), out);
  if (len) *len = n;
  if (seq_len) *seq_len = int32_t(s.len);
  return PA_OK;
}

pa_status pa_pack_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t num_seqs,
                               int32_t max_blocks, int32_t* tables_out, int32_t* lens_out) {
  if (!a || (!seq_ids && num_seqs > 0) || max_blocks < 0)
    return pa::fail(PA_ERR_INVALID, "pa_pack_block_tables: bad argument");
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return pa::fail(PA_ERR_NO_SEQ, "pa_pack_block_tables: no sequence %lld",
                      (long long)seq_ids[i]);
    if (int64_t(it->second.table.size()) > max_blocks)
      return pa::fail(PA_ERR_INVALID, "pa_pack_block_tables: sequence %lld has %zu blocks > %d",
                      (long long)seq_ids[i], it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = a->seqs.find(seq_ids[i])->second;
    if (tables_out) {
      int32_t* row = tables_out + int64_t(i) * max_blocks;
      size_t n = s.table.size();
      std::copy(s.table.begin(), s.table.end(), row);
      std::fill(row + n, row + max_blocks, -1);
    }
    if (lens_out) lens_out[i] = int32_t(s.len);
  }
  return PA_OK;
}

int32_t pa_num_free_blocks(const pa_allocator* a) { return a ? int32_t(a->count) : -1; }

int32_t pa_block_refcount(const pa_allocator* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->refs[block];
}

pa_status pa_allocator_stats(const pa_allocator* a, int64_t* out5) {
  if (!a || !out5) return pa::fail(PA_ERR_INVALID, "pa_allocator_stats: NULL argument");
  int64_t used = 0, shared = 0;
  for (int32_t r : a->refs) {
    used += r > 0;
    shared += r > 1;
  }
  out5[0] = used;
  out5[1] = shared;
  out5[2] = a->cow_copies;
  out5[3] = a->oom_refusals;
  out5[4] = int64_t(a->seqs.size());
  return PA_OK;
}

}  // extern "C"
