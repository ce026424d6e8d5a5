// Host allocator with a block size per request, behind the pa_buddy_* calls
// of pa.h.
//
// The first page's "3.0" feature: the block (page) size follows the
// request's length, blocks of different sizes serving requests of different
// lengths.  Built as one arena per layer, carved by a binary buddy system:
//
//  * the arena is a whole number of 64-token blocks; its unit is 8 tokens; a
//    block of 8 * 2^k tokens (order k = 0..3) is 2^k units starting at a
//    multiple of 2^k.  In the pool view of block size b the arena is
//    [arena_tokens / b][heads][b][head_dim], and block id i of that view is
//    units [i * b/8, (i+1) * b/8): a sequence's table indexes the view of
//    its own size, so the kernels run on each view unchanged;
//  * size rule: the largest size b with b <= n / 16 (at least 8) for a
//    request of n tokens, unless the caller names one; a sequence keeps its
//    size;
//  * one FIFO free list per order (intrusive doubly linked lists over unit
//    addresses, so that a merge can unlink a buddy in O(1)); a request for
//    order k takes the front of list k, else splits the front of the nearest
//    larger non-empty list, keeping the lower half and putting each upper
//    half at the back of the list below; a freed block merges with its buddy
//    (unit address XOR 2^k) while that buddy is free at the same order, then
//    goes to the back of its list;
//  * like the fixed-size allocator: per-block reference counts (fork,
//    copy-on-write of a shared, partly filled last block, taken before the
//    growth blocks), all or nothing with the whole demand counted first.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "status.h"

namespace {

constexpr int kOrders = 4;   // 8, 16, 32, 64 tokens
constexpr int kTop = kOrders - 1;
constexpr int kUnit = 8;
constexpr int kBlocksPerRequest = 16;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int order_of(int32_t bs) {
  for (int k = 0; k < kOrders; ++k)
    if (bs == (kUnit << k)) return k;
  return -1;
}

struct Seq {
  int order = 0;
  std::vector<int32_t> table;  // block ids in the view of this order
  int64_t len = 0;
};

}  // namespace

struct pa_buddy_allocator {
  int64_t units = 0;
  // Free lists: head/tail per order, prev/next per unit address; free_at[u]
  // is the order of the free block starting at u, or -1.
  int64_t head[kOrders], tail[kOrders], count[kOrders];
  std::vector<int64_t> prev, next;
  std::vector<int8_t> free_at;
  std::vector<int32_t> refs;  // per unit address of an allocated block
  std::unordered_map<int64_t, Seq> seqs;
  int64_t cow_copies = 0, oom_refusals = 0;

  void push_back(int64_t u, int k) {
    free_at[u] = int8_t(k);
    prev[u] = tail[k];
    next[u] = -1;
    if (tail[k] >= 0) next[tail[k]] = u; else head[k] = u;
    tail[k] = u;
    ++count[k];
  }
  void unlink(int64_t u) {
    const int k = free_at[u];
    if (prev[u] >= 0) next[prev[u]] = next[u]; else head[k] = next[u];
    if (next[u] >= 0) prev[next[u]] = prev[u]; else tail[k] = prev[u];
    free_at[u] = -1;
    --count[k];
  }
  int64_t obtainable(int k) const {
    int64_t n = 0;
    for (int j = k; j < kOrders; ++j) n += count[j] << (j - k);
    return n;
  }
  // Take one block of order k (obtainable(k) > 0 checked by the caller).
  int64_t take(int k) {
    int j = k;
    while (count[j] == 0) ++j;
    const int64_t a = head[j];
    unlink(a);
    while (j > k) {
      --j;
      push_back(a + (int64_t(1) << j), j);
    }
    refs[a] = 1;
    return a;
  }
  void give(int64_t a, int k) {
    while (k < kTop) {
      const int64_t b = a ^ (int64_t(1) << k);
      if (free_at[b] != k) break;
      unlink(b);
      a = std::min(a, b);
      ++k;
    }
    push_back(a, k);
  }
  void drop(int32_t id, int k) {
    const int64_t a = int64_t(id) << k;
    if (--refs[a] == 0) give(a, k);
  }
  int64_t slot(const Seq& s, int64_t pos) const {
    const int64_t bs = kUnit << s.order;
    return int64_t(s.table[pos / bs]) * bs + pos % bs;
  }
  // Blocks an append of n tokens needs, given its last block's reference
  // count; *cow tells whether a copy is part of it.
  int64_t demand(const Seq& s, int64_t n, int32_t last_refs, bool* cow) const {
    const int64_t bs = kUnit << s.order;
    *cow = n > 0 && s.len % bs != 0 && last_refs > 1;
    return ceil_div(s.len + n, bs) - ceil_div(s.len, bs) + (*cow ? 1 : 0);
  }
  void apply_append(Seq& s, int64_t n, int64_t* slots_out, int32_t* pair) {
    const int k = s.order;
    const int64_t bs = kUnit << k;
    pair[0] = pair[1] = -1;
    if (n > 0 && s.len % bs != 0 && refs[int64_t(s.table.back()) << k] > 1) {
      const int32_t src = s.table.back();
      const int32_t dst = int32_t(take(k) >> k);
      --refs[int64_t(src) << k];
      s.table.back() = dst;
      ++cow_copies;
      pair[0] = src;
      pair[1] = dst;
    }
    const int64_t grow = ceil_div(s.len + n, bs) - ceil_div(s.len, bs);
    for (int64_t i = 0; i < grow; ++i) s.table.push_back(int32_t(take(k) >> k));
    const int64_t start = s.len;
    s.len += n;
    if (slots_out)
      for (int64_t p = start; p < s.len; ++p) slots_out[p - start] = slot(s, p);
  }
};

extern "C" {

int32_t pa_buddy_size_for(int64_t num_tokens) {
  int32_t b = kUnit;
  for (int k = 0; k < kOrders; ++k)
    if (int64_t(kUnit << k) * kBlocksPerRequest <= num_tokens) b = kUnit << k;
  return b;
}

pa_status pa_buddy_create(int64_t arena_tokens, const int32_t* top_order, pa_buddy_allocator** out) {
  if (!out) return pa::fail(PA_ERR_INVALID, "pa_buddy_create: out is NULL");
  *out = nullptr;
  const int64_t top_tokens = int64_t(kUnit) << kTop;
  if (arena_tokens <= 0 || arena_tokens % top_tokens != 0 ||
      arena_tokens / kUnit > int64_t(INT32_MAX))
    return pa::fail(PA_ERR_INVALID,
                    "pa_buddy_create: arena_tokens %lld is not a positive multiple of %lld",
                    (long long)arena_tokens, (long long)top_tokens);
  pa_buddy_allocator* a = new (std::nothrow) pa_buddy_allocator();
  if (!a) return pa::fail(PA_ERR_OOM, "pa_buddy_create: host allocation failed");
  try {
    a->units = arena_tokens / kUnit;
    a->prev.assign(a->units, -1);
    a->next.assign(a->units, -1);
    a->free_at.assign(a->units, -1);
    a->refs.assign(a->units, 0);
  } catch (const std::bad_alloc&) {
    delete a;
    return pa::fail(PA_ERR_OOM, "pa_buddy_create: host allocation failed");
  }
  for (int k = 0; k < kOrders; ++k) a->head[k] = a->tail[k] = -1, a->count[k] = 0;
  const int64_t n_top = a->units >> kTop;
  if (top_order) {
    std::vector<char> seen(n_top, 0);
    for (int64_t i = 0; i < n_top; ++i) {
      const int32_t b = top_order[i];
      if (b < 0 || b >= n_top || seen[b]) {
        delete a;
        return pa::fail(PA_ERR_INVALID, "pa_buddy_create: top_order is not a permutation");
      }
      seen[b] = 1;
    }
  }
  for (int64_t i = 0; i < n_top; ++i)
    a->push_back(int64_t(top_order ? top_order[i] : i) << kTop, kTop);
  *out = a;
  return PA_OK;
}

void pa_buddy_destroy(pa_buddy_allocator* a) { delete a; }

pa_status pa_buddy_alloc_prompt(pa_buddy_allocator* a, int64_t seq_id, int32_t num_tokens,
                                int32_t block_size, int32_t* block_size_out, int64_t* slots_out) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_buddy_alloc_prompt: allocator is NULL");
  if (num_tokens < 0) return pa::fail(PA_ERR_INVALID, "pa_buddy_alloc_prompt: num_tokens < 0");
  const int32_t bs = block_size == 0 ? pa_buddy_size_for(num_tokens) : block_size;
  const int k = order_of(bs);
  if (k < 0)
    return pa::fail(PA_ERR_INVALID, "pa_buddy_alloc_prompt: block size %d (8, 16, 32, 64)", bs);
  if (a->seqs.count(seq_id))
    return pa::fail(PA_ERR_INVALID, "pa_buddy_alloc_prompt: sequence %lld exists",
                    (long long)seq_id);
  const int64_t need = ceil_div(num_tokens, bs);
  if (need > a->obtainable(k)) {
    ++a->oom_refusals;
    return pa::fail(PA_ERR_OOM, "OOM: prompt needs %lld blocks of %d, %lld obtainable",
                    (long long)need, bs, (long long)a->obtainable(k));
  }
  try {
    Seq s;
    s.order = k;
    s.table.reserve(need);
    auto ins = a->seqs.emplace(seq_id, std::move(s));
    Seq& q = ins.first->second;
    for (int64_t i = 0; i < need; ++i) q.table.push_back(int32_t(a->take(k) >> k));
    q.len = num_tokens;
    if (slots_out)
      for (int64_t p = 0; p < num_tokens; ++p) slots_out[p] = a->slot(q, p);
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_OOM, "pa_buddy_alloc_prompt: host allocation failed");
  }
  if (block_size_out) *block_size_out = bs;
  return PA_OK;
}

pa_status pa_buddy_append_tokens(pa_buddy_allocator* a, int64_t seq_id, int32_t n,
                                 int64_t* slots_out, int32_t* cow_src_dst, int32_t* num_cow) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_buddy_append_tokens: allocator is NULL");
  if (n < 0) return pa::fail(PA_ERR_INVALID, "pa_buddy_append_tokens: n < 0");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_buddy_append_tokens: no sequence %lld", (long long)seq_id);
  Seq& s = it->second;
  if (s.len + n > INT32_MAX)   // lengths leave the allocator as int32
    return pa::fail(PA_ERR_INVALID,
                    "pa_buddy_append_tokens: sequence %lld would pass INT32_MAX tokens",
                    (long long)seq_id);
  bool cow = false;
  const int32_t last_refs = s.table.empty() ? 0 : a->refs[int64_t(s.table.back()) << s.order];
  const int64_t need = a->demand(s, n, last_refs, &cow);
  if (need > a->obtainable(s.order)) {
    ++a->oom_refusals;
    return pa::fail(PA_ERR_OOM, "OOM: append needs %lld blocks, %lld obtainable",
                    (long long)need, (long long)a->obtainable(s.order));
  }
  int32_t pair[2];
  try {
    s.table.reserve(s.table.size() + size_t(need));
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_OOM, "pa_buddy_append_tokens: host allocation failed");
  }
  a->apply_append(s, n, slots_out, pair);
  if (cow_src_dst) cow_src_dst[0] = pair[0], cow_src_dst[1] = pair[1];
  if (num_cow) *num_cow = pair[0] >= 0 ? 1 : 0;
  return PA_OK;
}

pa_status pa_buddy_append_tokens_batch(pa_buddy_allocator* a, const int64_t* seq_ids,
                                       int32_t num_seqs, int32_t n, int64_t* slots_out,
                                       int32_t* cow_pairs_out, int32_t* num_cow) {
  if (!a || (!seq_ids && num_seqs > 0))
    return pa::fail(PA_ERR_INVALID, "pa_buddy_append_tokens_batch: NULL argument");
  if (n < 0 || num_seqs < 0)
    return pa::fail(PA_ERR_INVALID, "pa_buddy_append_tokens_batch: negative size");
  std::vector<Seq*> listed;
  try {
    std::unordered_set<int64_t> ids;
    listed.reserve(num_seqs);
    for (int32_t i = 0; i < num_seqs; ++i) {
      if (!ids.insert(seq_ids[i]).second)
        return pa::fail(PA_ERR_INVALID, "pa_buddy_append_tokens_batch: sequence %lld listed twice",
                        (long long)seq_ids[i]);
      auto it = a->seqs.find(seq_ids[i]);
      if (it == a->seqs.end())
        return pa::fail(PA_ERR_NO_SEQ, "pa_buddy_append_tokens_batch: no sequence %lld",
                        (long long)seq_ids[i]);
      if (it->second.len + n > INT32_MAX)
        return pa::fail(PA_ERR_INVALID,
                        "pa_buddy_append_tokens_batch: sequence %lld would pass INT32_MAX tokens",
                        (long long)seq_ids[i]);
      listed.push_back(&it->second);
    }
    // Dry run on the free-list counts: the batch's takes in order (a take
    // of order k uses list k, else splits the nearest larger block, which
    // adds one block to every order in between).  A copy made for an
    // earlier sequence drops its reference, which a later sequence sharing
    // that block sees.
    int64_t c[kOrders];
    std::copy(a->count, a->count + kOrders, c);
    std::unordered_map<int64_t, int32_t> dropped;
    for (Seq* s : listed) {
      const int64_t last = s->table.empty() ? -1 : int64_t(s->table.back()) << s->order;
      const int32_t last_refs = last < 0 ? 0 : a->refs[last] - (dropped.count(last) ? dropped[last] : 0);
      bool cow = false;
      const int64_t need = a->demand(*s, n, last_refs, &cow);
      if (cow) ++dropped[last];
      for (int64_t i = 0; i < need; ++i) {
        int j = s->order;
        while (j < kOrders && c[j] == 0) ++j;
        if (j == kOrders) {
          ++a->oom_refusals;
          return pa::fail(PA_ERR_OOM, "OOM: batch append runs out of blocks of %d",
                          kUnit << s->order);
        }
        --c[j];
        for (int i2 = s->order; i2 < j; ++i2) ++c[i2];
      }
      s->table.reserve(s->table.size() + size_t(need));
    }
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_OOM, "pa_buddy_append_tokens_batch: host allocation failed");
  }
  int32_t copies = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    int32_t pair[2];
    a->apply_append(*listed[i], n, slots_out ? slots_out + int64_t(i) * n : nullptr, pair);
    if (cow_pairs_out) cow_pairs_out[2 * i] = pair[0], cow_pairs_out[2 * i + 1] = pair[1];
    if (pair[0] >= 0) ++copies;
  }
  if (num_cow) *num_cow = copies;
  return PA_OK;
}

pa_status pa_buddy_fork(pa_buddy_allocator* a, int64_t parent_id, int64_t child_id) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_buddy_fork: allocator is NULL");
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_buddy_fork: no sequence %lld", (long long)parent_id);
  if (a->seqs.count(child_id))
    return pa::fail(PA_ERR_INVALID, "pa_buddy_fork: sequence %lld exists", (long long)child_id);
  try {
    Seq child = it->second;
    for (int32_t b : child.table) ++a->refs[int64_t(b) << child.order];
    a->seqs.emplace(child_id, std::move(child));
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_OOM, "pa_buddy_fork: host allocation failed");
  }
  return PA_OK;
}

pa_status pa_buddy_free_seq(pa_buddy_allocator* a, int64_t seq_id) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_buddy_free_seq: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_buddy_free_seq: no sequence %lld", (long long)seq_id);
  for (int32_t b : it->second.table) a->drop(b, it->second.order);
  a->seqs.erase(it);
  return PA_OK;
}

pa_status pa_buddy_get_block_table(const pa_buddy_allocator* a, int64_t seq_id, int32_t* out,
                                   int32_t cap, int32_t* len, int32_t* seq_len,
                                   int32_t* block_size) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_buddy_get_block_table: allocator is NULL");
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_buddy_get_block_table: no sequence %lld",
                    (long long)seq_id);
  const Seq& s = it->second;
  const int32_t n = int32_t(s.table.size());
  if (out) std::copy_n(s.table.begin(), std::min(n, std::max(cap, 0)), out);
  if (len) *len = n;
  if (seq_len) *seq_len = int32_t(s.len);
  if (block_size) *block_size = kUnit << s.order;
  return PA_OK;
}

pa_status pa_buddy_pack_block_tables(const pa_buddy_allocator* a, const int64_t* seq_ids,
                                     int32_t num_seqs, int32_t max_blocks, int32_t* tables_out,
                                     int32_t* lens_out) {
  if (!a || (num_seqs > 0 && (!seq_ids || !tables_out || !lens_out)) || num_seqs < 0 ||
      max_blocks < 0)
    return pa::fail(PA_ERR_INVALID, "pa_buddy_pack_block_tables: bad argument");
  int order = -1;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end())
      return pa::fail(PA_ERR_NO_SEQ, "pa_buddy_pack_block_tables: no sequence %lld",
                      (long long)seq_ids[i]);
    if (order >= 0 && it->second.order != order)
      return pa::fail(PA_ERR_INVALID,
                      "pa_buddy_pack_block_tables: sequences of different block sizes");
    order = it->second.order;
    if (int64_t(it->second.table.size()) > max_blocks)
      return pa::fail(PA_ERR_INVALID, "pa_buddy_pack_block_tables: %zu blocks > max_blocks %d",
                      it->second.table.size(), max_blocks);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables_out + int64_t(i) * max_blocks;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks, -1);
    lens_out[i] = int32_t(s.len);
  }
  return PA_OK;
}

int64_t pa_buddy_free_tokens(const pa_buddy_allocator* a) {
  if (!a) return 0;
  int64_t n = 0;
  for (int k = 0; k < kOrders; ++k) n += a->count[k] << k;
  return n * kUnit;
}

pa_status pa_buddy_free_list(const pa_buddy_allocator* a, int32_t block_size, int32_t* out,
                             int32_t cap, int32_t* len) {
  if (!a) return pa::fail(PA_ERR_INVALID, "pa_buddy_free_list: allocator is NULL");
  const int k = order_of(block_size);
  if (k < 0) return pa::fail(PA_ERR_INVALID, "pa_buddy_free_list: block size %d", block_size);
  int32_t n = 0;
  for (int64_t u = a->head[k]; u >= 0; u = a->next[u], ++n)
    if (out && n < cap) out[n] = int32_t(u >> k);
  if (len) *len = n;
  return PA_OK;
}

int32_t pa_buddy_block_refcount(const pa_buddy_allocator* a, int32_t block_size, int32_t block_id) {
  const int k = order_of(block_size);
  if (!a || k < 0 || block_id < 0 || (int64_t(block_id) << k) >= a->units) return -1;
  return a->refs[int64_t(block_id) << k];
}

}  // extern "C"
