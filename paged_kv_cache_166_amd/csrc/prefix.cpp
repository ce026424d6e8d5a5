// Prefix index over token ids behind the pa_prefix_* calls of pa.h.
//
// The DataWhale notes' RadixAttention section: cached token sequences kept in
// a radix (compressed prefix) tree whose edges hold runs of tokens and whose
// nodes point at the physical KV blocks; a new prompt is matched from the
// root by longest common prefix, the matched part reuses its blocks and only
// the unmatched suffix is computed; a node is split where a new sequence
// leaves the middle of an edge.
//
// Blocks: each inserted sequence is an entry with its block table.  An entry
// provides the positions from its divergence point d (its match length
// before insertion) to its end, and holds one allocator reference on each of
// its blocks that covers one of them (indices d / bs .. (n-1) / bs), so
// cached blocks outlive their sequence.  Every tree node remembers the entry
// that created its positions (a split keeps it on both halves); block j of a
// hit of h tokens comes from the creator of the node holding position
// min((j+1) bs, h) - 1, the last hit position in that block -- an entry whose
// tokens equal the prompt up to there, so its block j holds the right rows.
// A hit that ends inside a block shares that partly filled block; the
// allocator's copy-on-write copies it on the sequence's first write.
//
// Eviction (the notes' LRU rule: when memory is full, the KV cache of leaf
// nodes goes first, least recently used first, until there is room): every
// insertion and cached-prompt allocation stamps the nodes its walk entered
// with a logical clock; a leaf is evicted whole, oldest stamp first (ties to
// the older node); evicting it drops its creator's references on the blocks
// only it uses -- the block under its first position stays when the parent
// node has the same creator and also lies in it -- and blocks left with no
// reference go back to the free list.  Live sequences keep their own
// references, so eviction never takes their blocks.  With automatic eviction
// switched on, an allocation that would run out evicts until it fits, on an
// undo log: if evicting every leaf (but those of a cached prompt's own hit)
// is not enough, the evictions are undone and the call fails unchanged.
#include <algorithm>
#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
#include <unordered_set>
#include <utility>
#include <vector>

#include "allocator_impl.h"
#include "pa.h"
#include "status.h"

namespace {

struct Node {
  std::vector<int32_t> edge;  // tokens on the edge into this node
  int64_t start = 0;          // depth of edge[0]
  int32_t creator = -1;       // entry whose insertion created these positions
  int32_t parent = -1;
  uint64_t stamp = 0;         // clock of the last walk that entered it
  bool alive = true;          // false once evicted (ids are never reused)
  std::unordered_map<int32_t, int32_t> kids;  // first token of a child's edge -> node
  int64_t end() const { return start + int64_t(edge.size()); }
};

struct Entry {
  std::vector<int32_t> table;  // the sequence's blocks covering its n tokens
  int64_t ref_base = 0;        // block index of refs[0]
  std::vector<int32_t> refs;   // block referenced at each index from ref_base, -1 once dropped
  int64_t held = 0;            // references still held
  int32_t live_nodes = 0;      // live tree nodes this entry created (0: nothing uses it)
};

// What one eviction changed, so that a failed reclaim can put it back.
struct Evicted {
  int32_t leaf;
  bool parent_became_leaf;
  std::vector<std::pair<int64_t, int32_t>> released;  // (block index, block), in order
};

// One step of a walk: node, and the depth range [lo, hi) of the prompt it
// matched along that node's edge.
struct Seg {
  int32_t node;
  int64_t lo, hi;
};

}  // namespace

struct pa_prefix_index {
  pa_allocator* alloc = nullptr;
  std::vector<Node> nodes;  // nodes[0] is the root (empty edge)
  std::vector<Entry> entries;
  std::set<std::pair<uint64_t, int32_t>> leaves;  // (stamp, node) of every live leaf
  uint64_t clock = 0;
  int64_t evicted = 0;
  int64_t inserted = 0;   // entries inserted since creation or the last clear
  int64_t live = 1;       // live nodes (the root included)

  bool is_leaf(int32_t id) const { return id != 0 && nodes[id].alive && nodes[id].kids.empty(); }

  void touch(int32_t id) {
    if (is_leaf(id)) {
      leaves.erase({nodes[id].stamp, id});
      leaves.insert({clock, id});
    }
    nodes[id].stamp = clock;
  }

  // Longest match of tokens from the root; the segments walked, and where
  // the walk stopped (node, offset in its edge) for an insertion.
  int64_t walk(const int32_t* t, int64_t n, std::vector<Seg>* segs, int32_t* stop_node,
               int64_t* stop_off) const {
    int32_t cur = 0;
    int64_t depth = 0;
    if (stop_node) *stop_node = 0;
    if (stop_off) *stop_off = 0;
    while (depth < n) {
      const Node& c = nodes[cur];
      auto it = c.kids.find(t[depth]);
      if (it == c.kids.end()) break;
      const Node& k = nodes[it->second];
      int64_t m = 0;
      while (m < int64_t(k.edge.size()) && depth + m < n && k.edge[m] == t[depth + m]) ++m;
      if (segs) segs->push_back({it->second, depth, depth + m});
      depth += m;
      if (m < int64_t(k.edge.size())) {  // stopped inside this edge
        if (stop_node) *stop_node = it->second;
        if (stop_off) *stop_off = m;
        return depth;
      }
      cur = it->second;
      if (stop_node) *stop_node = cur;
      if (stop_off) *stop_off = int64_t(k.edge.size());
    }
    return depth;
  }

  // Blocks of a hit of h tokens along the segments of its walk.
  void hit_blocks(const std::vector<Seg>& segs, int64_t h, std::vector<int32_t>* out) const {
    const int32_t bs = alloc->block_size;
    size_t s = 0;
    for (int64_t j = 0; j < pa_alloc::blocks_for(h, bs); ++j) {
      const int64_t q = std::min<int64_t>((j + 1) * bs, h) - 1;
      while (segs[s].hi <= q) ++s;
      out->push_back(entries[nodes[segs[s].node].creator].table[j]);
    }
  }

  void release(int32_t b) {
    if (--alloc->refs[b] == 0) alloc->give_back(b);
  }

  // Oldest live leaf not in keep, or -1.
  int32_t oldest(const std::unordered_set<int32_t>& keep) const {
    for (const auto& l : leaves)
      if (!keep.count(l.second)) return l.second;
    return -1;
  }

  Evicted evict(int32_t id) {
    Node& L = nodes[id];
    Node& P = nodes[L.parent];
    Entry& e = entries[L.creator];
    const int32_t bs = alloc->block_size;
    int64_t first = L.start / bs;
    if (L.start % bs != 0 && L.parent != 0 && P.creator == L.creator) ++first;
    const int64_t last = (L.end() - 1) / bs;
    Evicted r{id, false, {}};
    r.released.reserve(size_t(std::max<int64_t>(last - first + 1, 0)));
    const bool parent_leaf = L.parent != 0 && P.kids.size() == 1;
    if (parent_leaf) leaves.insert({P.stamp, L.parent});
    for (int64_t j = std::max(first, e.ref_base); j <= last; ++j) {
      const int64_t k = j - e.ref_base;
      if (k >= int64_t(e.refs.size()) || e.refs[k] < 0) continue;
      const int32_t b = e.refs[k];
      e.refs[k] = -1;
      --e.held;
      r.released.emplace_back(j, b);
      release(b);
    }
    leaves.erase({L.stamp, id});
    P.kids.erase(L.edge[0]);
    L.alive = false;
    --e.live_nodes;
    --live;
    r.parent_became_leaf = parent_leaf;
    return r;
  }

  void undo(const Evicted& r) {
    Node& L = nodes[r.leaf];
    Node& P = nodes[L.parent];
    Entry& e = entries[L.creator];
    if (r.parent_became_leaf) leaves.erase({P.stamp, L.parent});
    L.alive = true;
    ++e.live_nodes;
    ++live;
    P.kids[L.edge[0]] = r.leaf;
    leaves.insert({L.stamp, r.leaf});
    for (auto it = r.released.rbegin(); it != r.released.rend(); ++it) {
      const int32_t b = it->second;
      if (alloc->refs[b] == 0) --alloc->count;  // it was the free list's last entry
      ++alloc->refs[b];
      e.refs[it->first - e.ref_base] = b;
      ++e.held;
    }
  }

  // Evicted nodes keep their ids (ties go to the older node) and entries
  // their numbers; once the dead outnumber the live nodes (plus a margin),
  // both are renumbered in order, dropping the dead nodes and the entries no
  // live node uses (they hold no reference any more).  Order is all that the
  // ids decide, so nothing observable changes.  Never called while node ids
  // are held (a walk's segments, an undo log).
  void maybe_compact() {
    const int64_t dead = int64_t(nodes.size()) - live;
    if (dead <= live + 64) return;
    try {
      std::vector<int32_t> emap(entries.size(), -1), nmap(nodes.size(), -1);
      std::vector<Entry> ne;
      std::vector<Node> nn;
      int32_t k = 0;
      for (size_t i = 0; i < entries.size(); ++i)
        if (entries[i].live_nodes > 0) emap[i] = k++;
      ne.reserve(size_t(k));
      k = 0;
      for (size_t i = 0; i < nodes.size(); ++i)
        if (nodes[i].alive) nmap[i] = k++;
      nn.reserve(size_t(k));
      for (size_t i = 0; i < entries.size(); ++i)
        if (emap[i] >= 0) ne.push_back(std::move(entries[i]));
      for (size_t i = 0; i < nodes.size(); ++i) {
        if (nmap[i] < 0) continue;
        Node nd = std::move(nodes[i]);
        nd.parent = nd.parent >= 0 ? nmap[nd.parent] : -1;
        nd.creator = nd.creator >= 0 ? emap[nd.creator] : -1;
        for (auto& kv : nd.kids) kv.second = nmap[kv.second];
        nn.push_back(std::move(nd));
      }
      std::set<std::pair<uint64_t, int32_t>> nl;
      for (const auto& lf : leaves) nl.insert({lf.first, nmap[lf.second]});
      entries.swap(ne);
      nodes.swap(nn);
      leaves.swap(nl);
    } catch (const std::bad_alloc&) {
      // the index is untouched until the swaps: keep it as it is
    }
  }

  // Evict oldest leaves outside keep until fits(); all or nothing.
  bool reclaim(const std::function<bool()>& fits, const std::unordered_set<int32_t>& keep) {
    std::vector<Evicted> log;
    try {
      while (!fits()) {
        const int32_t id = oldest(keep);
        if (id < 0) break;
        log.emplace_back();  // room first: evict() itself leaves nothing half done
        log.back() = evict(id);
      }
    } catch (const std::bad_alloc&) {
      for (auto it = log.rbegin(); it != log.rend(); ++it) undo(*it);
      return false;
    }
    if (fits()) {
      evicted += int64_t(log.size());
      return true;
    }
    for (auto it = log.rbegin(); it != log.rend(); ++it) undo(*it);
    return false;
  }
};

bool pa_alloc::reclaim(pa_prefix_index* x, const std::function<bool()>& fits) {
  const bool ok = x->reclaim(fits, {});
  x->maybe_compact();
  return ok;
}

extern "C" {

pa_status pa_prefix_index_create(pa_allocator* a, pa_prefix_index** out) {
  if (!out || !a) return pa::fail(PA_ERR_INVALID, "pa_prefix_index_create: NULL argument");
  *out = nullptr;
  pa_prefix_index* x = new (std::nothrow) pa_prefix_index();
  if (!x) return pa::fail(PA_ERR_OOM, "pa_prefix_index_create: host allocation failed");
  x->alloc = a;
  x->nodes.emplace_back();
  *out = x;
  return PA_OK;
}

pa_status pa_prefix_clear(pa_prefix_index* x) {
  if (!x) return pa::fail(PA_ERR_INVALID, "pa_prefix_clear: index is NULL");
  for (const Entry& e : x->entries)
    for (int32_t b : e.refs)
      if (b >= 0) x->release(b);
  x->entries.clear();
  x->nodes.clear();
  x->nodes.emplace_back();
  x->leaves.clear();
  x->inserted = 0;
  x->live = 1;
  return PA_OK;
}

void pa_prefix_index_destroy(pa_prefix_index* x) {
  if (!x) return;
  if (x->alloc->evictor == x) x->alloc->evictor = nullptr;
  pa_prefix_clear(x);
  delete x;
}

pa_status pa_prefix_insert(pa_prefix_index* x, int64_t seq_id, const int32_t* tokens,
                           int32_t num_tokens, int32_t* divergence) {
  if (!x || (!tokens && num_tokens > 0) || num_tokens < 0)
    return pa::fail(PA_ERR_INVALID, "pa_prefix_insert: bad argument");
  pa_allocator* a = x->alloc;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end())
    return pa::fail(PA_ERR_NO_SEQ, "pa_prefix_insert: no sequence %lld", (long long)seq_id);
  const pa_alloc::Sequence& s = it->second;
  if (num_tokens > s.len)
    return pa::fail(PA_ERR_INVALID, "pa_prefix_insert: %d tokens, sequence holds %lld",
                    num_tokens, (long long)s.len);
  const int32_t bs = a->block_size;
  const int64_t n = num_tokens;
  try {
    int32_t stop_node = 0;
    int64_t stop_off = 0;
    std::vector<Seg> segs;
    const int64_t d = x->walk(tokens, n, &segs, &stop_node, &stop_off);
    Entry e;
    e.table.assign(s.table.begin(), s.table.begin() + pa_alloc::blocks_for(n, bs));
    if (d < n) {
      e.ref_base = d / bs;
      for (int64_t j = d / bs; j <= (n - 1) / bs; ++j) e.refs.push_back(e.table[j]);
    }
    e.held = int64_t(e.refs.size());
    const int32_t eid = int32_t(x->entries.size());
    x->nodes.reserve(x->nodes.size() + 2);
    x->entries.reserve(x->entries.size() + 1);
    ++x->clock;
    for (const Seg& g : segs) x->touch(g.node);
    if (d < n) {
      int32_t parent = stop_node;
      if (stop_node != 0 && stop_off < int64_t(x->nodes[stop_node].edge.size())) {
        // Split the edge: a new upper node keeps edge[0, off) and the creator.
        Node& low = x->nodes[stop_node];
        Node up;
        up.edge.assign(low.edge.begin(), low.edge.begin() + stop_off);
        up.start = low.start;
        up.creator = low.creator;
        up.parent = low.parent;
        up.stamp = low.stamp;
        ++x->entries[low.creator].live_nodes;
        ++x->live;
        const int32_t up_id = int32_t(x->nodes.size());
        x->nodes[low.parent].kids[low.edge[0]] = up_id;  // the parent's link now points at up
        up.kids[low.edge[stop_off]] = stop_node;
        low.parent = up_id;
        low.edge.erase(low.edge.begin(), low.edge.begin() + stop_off);
        low.start += stop_off;
        x->nodes.push_back(std::move(up));
        parent = up_id;
      }
      Node leaf;
      leaf.edge.assign(tokens + d, tokens + n);
      leaf.start = d;
      leaf.creator = eid;
      leaf.parent = parent;
      leaf.stamp = x->clock;
      const int32_t leaf_id = int32_t(x->nodes.size());
      if (x->is_leaf(parent)) x->leaves.erase({x->nodes[parent].stamp, parent});
      x->nodes.push_back(std::move(leaf));
      x->nodes[parent].kids[tokens[d]] = leaf_id;
      x->leaves.insert({x->clock, leaf_id});
      e.live_nodes = 1;
      ++x->live;
    }
    for (int32_t b : e.refs) ++a->refs[b];
    // An entry that adds no position (all of it already cached) creates no
    // node and holds no reference: nothing will ever read it, so it is
    // counted but not kept.
    if (d < n) x->entries.push_back(std::move(e));
    ++x->inserted;
    if (divergence) *divergence = int32_t(d);
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_OOM, "pa_prefix_insert: host allocation failed");
  }
  return PA_OK;
}

pa_status pa_prefix_match(const pa_prefix_index* x, const int32_t* tokens, int32_t num_tokens,
                          int32_t* hit_len) {
  if (!x || !hit_len || (!tokens && num_tokens > 0) || num_tokens < 0)
    return pa::fail(PA_ERR_INVALID, "pa_prefix_match: bad argument");
  *hit_len = int32_t(x->walk(tokens, num_tokens, nullptr, nullptr, nullptr));
  return PA_OK;
}

pa_status pa_alloc_prompt_cached(pa_prefix_index* x, int64_t seq_id, const int32_t* tokens,
                                 int32_t num_tokens, int32_t* hit_len, int64_t* slots_out,
                                 int32_t* cow_src_dst, int32_t* num_cow) {
  if (!x || (!tokens && num_tokens > 0) || num_tokens < 0)
    return pa::fail(PA_ERR_INVALID, "pa_alloc_prompt_cached: bad argument");
  pa_allocator* a = x->alloc;
  if (a->seqs.count(seq_id))
    return pa::fail(PA_ERR_INVALID, "pa_alloc_prompt_cached: sequence %lld exists",
                    (long long)seq_id);
  const int32_t bs = a->block_size;
  try {
    std::vector<Seg> segs;
    const int64_t h = x->walk(tokens, num_tokens, &segs, nullptr, nullptr);
    const bool cow = num_tokens > h && h % bs != 0;
    const int64_t need = pa_alloc::blocks_for(num_tokens, bs) - pa_alloc::blocks_for(h, bs) +
                         (cow ? 1 : 0);
    ++x->clock;
    bool short_of = need > a->count;
    if (short_of && a->evictor == x) {
      std::unordered_set<int32_t> hit_nodes;
      for (const Seg& g : segs) hit_nodes.insert(g.node);
      short_of = !x->reclaim([&] { return need <= a->count; }, hit_nodes);
    }
    if (short_of) {
      ++a->oom_refusals;
      return pa::fail(PA_ERR_OOM, "OOM: cached prompt needs %lld blocks, %lld free",
                      (long long)need, (long long)a->count);
    }
    for (const Seg& g : segs) x->touch(g.node);
    pa_alloc::Sequence s;
    x->hit_blocks(segs, h, &s.table);
    s.table.reserve(pa_alloc::blocks_for(num_tokens, bs) + 1);
    s.len = h;
    auto ins = a->seqs.emplace(seq_id, std::move(s));
    for (int32_t b : ins.first->second.table) ++a->refs[b];
    int32_t pair[2];
    a->apply_append(ins.first->second, num_tokens - h, slots_out, pair);
    if (cow_src_dst) {
      cow_src_dst[0] = pair[0];
      cow_src_dst[1] = pair[1];
    }
    if (num_cow) *num_cow = pair[0] >= 0 ? 1 : 0;
    if (hit_len) *hit_len = int32_t(h);
  } catch (const std::bad_alloc&) {
    return pa::fail(PA_ERR_OOM, "pa_alloc_prompt_cached: host allocation failed");
  }
  x->maybe_compact();
  return PA_OK;
}

pa_status pa_prefix_stats(const pa_prefix_index* x, int64_t* out5) {
  if (!x || !out5) return pa::fail(PA_ERR_INVALID, "pa_prefix_stats: NULL argument");
  int64_t refs = 0;
  for (const Entry& e : x->entries) refs += e.held;
  out5[0] = x->inserted;
  out5[1] = x->live;
  out5[2] = refs;
  out5[3] = x->evicted;
  out5[4] = int64_t(x->nodes.size());
  return PA_OK;
}

pa_status pa_prefix_set_auto_evict(pa_prefix_index* x, int32_t enable) {
  if (!x) return pa::fail(PA_ERR_INVALID, "pa_prefix_set_auto_evict: index is NULL");
  pa_allocator* a = x->alloc;
  if (enable) {
    if (a->evictor && a->evictor != x)
      return pa::fail(PA_ERR_INVALID,
                      "pa_prefix_set_auto_evict: the allocator already has an evicting index");
    a->evictor = x;
  } else if (a->evictor == x) {
    a->evictor = nullptr;
  }
  return PA_OK;
}

pa_status pa_prefix_evict(pa_prefix_index* x, int64_t min_free_blocks, int64_t* num_evicted) {
  if (!x) return pa::fail(PA_ERR_INVALID, "pa_prefix_evict: index is NULL");
  int64_t n = 0;
  try {
    const std::unordered_set<int32_t> none;
    while (x->alloc->count < min_free_blocks) {
      const int32_t id = x->oldest(none);
      if (id < 0) break;
      x->evict(id);
      ++n;
    }
  } catch (const std::bad_alloc&) {
    x->evicted += n;
    if (num_evicted) *num_evicted = n;
    return pa::fail(PA_ERR_OOM, "pa_prefix_evict: host allocation failed");
  }
  x->evicted += n;
  if (num_evicted) *num_evicted = n;
  x->maybe_compact();
  return PA_OK;
}

}  // extern "C"
