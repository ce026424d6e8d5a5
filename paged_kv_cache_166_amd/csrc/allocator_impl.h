// The host allocator's state, shared by allocator.cpp (the pa_allocator_* /
// pa_alloc_* calls) and prefix.cpp (the prefix index, which takes and drops
// block references through it).  Not part of the C ABI.
#pragma once
#include <cstdint>
#include <functional>
#include <unordered_map>
#include <vector>

struct pa_prefix_index;

namespace pa_alloc {

inline int64_t blocks_for(int64_t tokens, int32_t bs) { return (tokens + bs - 1) / bs; }

struct Sequence {
  std::vector<int32_t> table;
  int64_t len = 0;
};

// Evicts the index's least recently used leaves until fits() holds; when
// evicting every leaf would not be enough, undoes what it evicted and
// returns false (defined with the index, prefix.cpp).
bool reclaim(pa_prefix_index* x, const std::function<bool()>& fits);

}  // namespace pa_alloc

struct pa_allocator {
  using Sequence = pa_alloc::Sequence;
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ring;  // free list, FIFO
  int64_t head = 0;
  int64_t count = 0;
  std::vector<int32_t> refs;
  std::unordered_map<int64_t, Sequence> seqs;
  int64_t cow_copies = 0;
  int64_t oom_refusals = 0;
  // A prefix index with automatic eviction switched on: an allocation that
  // would run out asks it to evict cached prefixes first.
  pa_prefix_index* evictor = nullptr;

  // True when an operation cannot get its blocks.  demand() is the operation's
  // need in the current state; an eviction can lower it (a last block that
  // loses the index's reference needs no copy), so it is asked again after
  // every eviction.
  bool short_of(const std::function<int64_t()>& demand) {
    if (demand() <= count) return false;
    return !evictor || !pa_alloc::reclaim(evictor, [&] { return demand() <= count; });
  }

  int32_t take() {
    int32_t b = ring[head];
    head = (head + 1) % num_blocks;
    --count;
    refs[b] = 1;
    return b;
  }
  void give_back(int32_t b) {
    ring[(head + count) % num_blocks] = b;
    ++count;
  }
  int64_t slot(const Sequence& s, int64_t pos) const {
    return int64_t(s.table[pos / block_size]) * block_size + pos % block_size;
  }
  // Blocks one append of n tokens to s needs, given the reference count its
  // last block has at that moment; *cow tells whether a copy is part of it.
  int64_t demand(const Sequence& s, int64_t n, int32_t last_refs, bool* cow) const {
    *cow = n > 0 && s.len % block_size != 0 && last_refs > 1;
    return pa_alloc::blocks_for(s.len + n, block_size) - pa_alloc::blocks_for(s.len, block_size) + (*cow ? 1 : 0);
  }
  // Apply an append whose demand has been checked.
  void apply_append(Sequence& s, int64_t n, int64_t* slots_out, int32_t* cow_pair) {
    bool cow = n > 0 && s.len % block_size != 0 && refs[s.table.back()] > 1;
    if (cow_pair) cow_pair[0] = cow_pair[1] = -1;
    if (cow) {
      int32_t src = s.table.back();
      int32_t dst = take();
      --refs[src];
      s.table.back() = dst;
      ++cow_copies;
      if (cow_pair) {
        cow_pair[0] = src;
        cow_pair[1] = dst;
      }
    }
    int64_t grow = pa_alloc::blocks_for(s.len + n, block_size) - pa_alloc::blocks_for(s.len, block_size);
    for (int64_t i = 0; i < grow; ++i) s.table.push_back(take());
    int64_t start = s.len;
    s.len += n;
    if (slots_out)
      for (int64_t p = start; p < s.len; ++p) slots_out[p - start] = slot(s, p);
  }
};

