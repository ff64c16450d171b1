// Host block allocator with a radix prefix cache (C ABI in include/pagedkv.h).
//
// "The radix prefix cache" (pyshine walkthrough of text-generation-inference v3):
// block 0 is kept back; free blocks sit in a free list; cached prefixes live in a
// compressed radix tree keyed by token ids at block granularity.  An allocation
// walks the tree with the request's prompt, takes a reference on the deepest
// matched node before anything can be evicted, then takes fresh blocks for the
// rest of the request, evicting least-recently-used unreferenced prefixes when the
// free list runs dry.  Freeing drops the reference and inserts the computed
// prefix into the tree, splitting an edge where the new tokens diverge; blocks of
// the request that another request cached meanwhile go back to the free list.
// "Inside the batching task": a prompt always keeps at least one token to compute.
// "Under the Hood: PagedAttention" (Text Generation Inference page), "Prefix
// sharing": shared blocks are copied before a write (copy-on-write); here fork()
// shares a request's blocks and prepare_write() hands out the copy.
//
// Choices where the pages say nothing: whole blocks only; the lowest free block id
// first; a clock advanced by every operation that can change recency, eviction of
// whole unreferenced leaves in (last use, creation) order; a per-block holder count
// (live allocations plus the tree).  Host code only; not thread-safe.
#include <stdint.h>

#include <algorithm>
#include <functional>
#include <map>
#include <queue>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

using Key = std::vector<int32_t>;   // the token ids of one block

struct TreeNode {
  std::vector<Key> keys;            // the blocks on the edge into this node
  std::vector<int32_t> blocks;      // their physical blocks
  std::map<Key, int> children;      // first key of a child's edge -> node index
  int parent = -1;
  int refs = 0;                     // allocations whose match ends here
  uint64_t last = 0;                // clock of the last use
  int64_t serial = 0;               // creation order (eviction tie-break)
  bool alive = true;
};

struct Allocation {
  std::vector<int32_t> blocks;
  int node = 0;                     // deepest matched node (0 = none)
};

struct Match {
  int node;                         // last node entered
  int depth;                        // blocks of its edge that matched
  int matched;                      // blocks matched in total
  std::vector<int> path;            // nodes entered, root excluded
};

}  // namespace

struct pkv_allocator {
  int32_t num_blocks, bs;
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_list;
  std::vector<int32_t> holders;
  std::vector<TreeNode> nodes;      // nodes[0] is the root
  std::unordered_map<int64_t, Allocation> allocs;
  uint64_t clock = 0;
  int64_t next_serial = 1, next_id = 1;

  pkv_allocator(int32_t nb, int32_t b) : num_blocks(nb), bs(b), holders(nb, 0) {
    for (int32_t i = 1; i < nb; ++i) free_list.push(i);
    nodes.emplace_back();
  }

  std::vector<Key> keys_of(const int32_t* tokens, int n_blocks) const {
    std::vector<Key> k((size_t)n_blocks);
    for (int i = 0; i < n_blocks; ++i) k[i].assign(tokens + (size_t)i * bs, tokens + (size_t)(i + 1) * bs);
    return k;
  }

  Match walk(const std::vector<Key>& keys) const {
    Match m{0, 0, 0, {}};
    int node = 0;
    while (m.matched < (int)keys.size()) {
      auto it = nodes[node].children.find(keys[m.matched]);
      if (it == nodes[node].children.end()) break;
      const int child = it->second;
      const TreeNode& c = nodes[child];
      int d = 0;
      while (d < (int)c.keys.size() && m.matched < (int)keys.size() && c.keys[d] == keys[m.matched]) {
        ++d;
        ++m.matched;
      }
      m.path.push_back(child);
      if (d < (int)c.keys.size()) {
        m.node = child;
        m.depth = d;
        return m;
      }
      node = child;
    }
    m.node = node;
    m.depth = (int)nodes[node].keys.size();
    return m;
  }

  // Cut node's edge after d blocks: a new parent takes the first d, node keeps the rest
  // (and its references and children).  Returns the node that ends after d blocks.
  int split(int node, int d) {
    if (d == 0 || d == (int)nodes[node].keys.size()) return node;
    TreeNode top;
    top.keys.assign(nodes[node].keys.begin(), nodes[node].keys.begin() + d);
    top.blocks.assign(nodes[node].blocks.begin(), nodes[node].blocks.begin() + d);
    top.parent = nodes[node].parent;
    top.last = nodes[node].last;
    top.serial = next_serial++;
    const int t = (int)nodes.size();
    nodes.push_back(std::move(top));
    TreeNode& n = nodes[node];
    nodes[n.parent].children[n.keys[0]] = t;
    n.keys.erase(n.keys.begin(), n.keys.begin() + d);
    n.blocks.erase(n.blocks.begin(), n.blocks.begin() + d);
    n.parent = t;
    nodes[t].children[n.keys[0]] = node;
    return t;
  }

  void release(int32_t b) {
    if (--holders[b] == 0) free_list.push(b);
  }

  // Evict unreferenced leaves, least recently used first, until `need` blocks are free.
  bool evict_until(size_t need) {
    while (free_list.size() < need) {
      int victim = -1;
      for (int i = 1; i < (int)nodes.size(); ++i) {
        const TreeNode& n = nodes[i];
        if (!n.alive || !n.children.empty() || n.refs != 0) continue;
        if (victim < 0 || n.last < nodes[victim].last ||
            (n.last == nodes[victim].last && n.serial < nodes[victim].serial))
          victim = i;
      }
      if (victim < 0) return false;
      TreeNode& v = nodes[victim];
      nodes[v.parent].children.erase(v.keys[0]);
      v.alive = false;
      for (int32_t b : v.blocks) release(b);
      v.keys.clear();
      v.blocks.clear();
    }
    return true;
  }

  std::vector<int32_t> take(size_t count) {
    std::vector<int32_t> out;
    out.reserve(count);
    for (size_t i = 0; i < count; ++i) {
      out.push_back(free_list.top());
      free_list.pop();
    }
    return out;
  }

  int32_t cached_blocks() const {
    int32_t c = 0;
    for (const TreeNode& n : nodes)
      if (n.alive) c += (int32_t)n.blocks.size();
    return c;
  }
};

namespace {

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

int copy_out(const std::vector<int32_t>& v, int32_t* out, int32_t capacity, int32_t* n_out) {
  if (n_out) *n_out = (int32_t)v.size();
  if (!out) return PKV_OK;
  if ((int32_t)v.size() > capacity) return PKV_EINVAL;
  std::copy(v.begin(), v.end(), out);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_allocator* pkv_allocator_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 2 || block_size < 1) return nullptr;
  try {
    return new pkv_allocator(num_blocks, block_size);
  } catch (...) {
    return nullptr;
  }
}

void pkv_allocator_destroy(pkv_allocator* a) { delete a; }

int pkv_allocator_allocate(pkv_allocator* a, const int32_t* tokens, int32_t n_tokens, int32_t n_total,
                           int64_t* alloc_id, int32_t* blocks, int32_t capacity, int32_t* n_blocks,
                           int32_t* prefix_len) {
  if (!a || !alloc_id || !blocks || !n_blocks || !prefix_len || n_tokens < 0 || n_total < 1 ||
      n_total < n_tokens || (n_tokens > 0 && !tokens))
    return PKV_EINVAL;
  const int32_t total_blocks = blocks_for(n_total, a->bs);
  if (capacity < total_blocks) return PKV_EINVAL;
  a->clock += 1;
  const int want = n_tokens > 0 ? (n_tokens - 1) / a->bs : 0;
  const std::vector<Key> keys = a->keys_of(tokens, want);
  const Match m = a->walk(keys);
  const int node = m.depth < (int)a->nodes[m.node].keys.size() ? a->split(m.node, m.depth) : m.node;
  std::vector<int> chain;
  for (int n = node; n != 0; n = a->nodes[n].parent) chain.push_back(n);
  std::reverse(chain.begin(), chain.end());
  std::vector<int32_t> out;
  for (int n : chain) out.insert(out.end(), a->nodes[n].blocks.begin(), a->nodes[n].blocks.end());
  if (node != 0) a->nodes[node].refs += 1;           // before anything can be evicted
  for (int n : chain) a->nodes[n].last = a->clock;
  const size_t fresh = (size_t)(total_blocks - m.matched);
  if (!a->evict_until(fresh)) {
    if (node != 0) a->nodes[node].refs -= 1;
    return PKV_ENOSPACE;
  }
  const std::vector<int32_t> fresh_blocks = a->take(fresh);
  out.insert(out.end(), fresh_blocks.begin(), fresh_blocks.end());
  for (int32_t b : out) a->holders[b] += 1;
  const int64_t id = a->next_id++;
  a->allocs[id] = Allocation{out, node};
  *alloc_id = id;
  *prefix_len = m.matched * a->bs;
  return copy_out(out, blocks, capacity, n_blocks);
}

int pkv_allocator_free(pkv_allocator* a, int64_t alloc_id, const int32_t* tokens, int32_t n_tokens) {
  if (!a || n_tokens < 0 || (n_tokens > 0 && !tokens)) return PKV_EINVAL;
  auto it = a->allocs.find(alloc_id);
  if (it == a->allocs.end()) return PKV_EINVAL;
  const Allocation al = it->second;
  a->allocs.erase(it);
  a->clock += 1;
  const int n_full = std::min<int>(n_tokens / a->bs, (int)al.blocks.size());
  const std::vector<Key> keys = a->keys_of(tokens, n_full);
  const Match m = a->walk(keys);
  for (int n : m.path) a->nodes[n].last = a->clock;
  if (m.matched < n_full) {
    const int parent = m.depth < (int)a->nodes[m.node].keys.size() ? a->split(m.node, m.depth) : m.node;
    TreeNode leaf;
    leaf.keys.assign(keys.begin() + m.matched, keys.end());
    leaf.blocks.assign(al.blocks.begin() + m.matched, al.blocks.begin() + n_full);
    leaf.parent = parent;
    leaf.last = a->clock;
    leaf.serial = a->next_serial++;
    for (int32_t b : leaf.blocks) a->holders[b] += 1;   // the tree holds them now
    const int li = (int)a->nodes.size();
    a->nodes[parent].children[leaf.keys[0]] = li;
    a->nodes.push_back(std::move(leaf));
  }
  if (al.node != 0) a->nodes[al.node].refs -= 1;
  for (int32_t b : al.blocks) a->release(b);
  return PKV_OK;
}

int pkv_allocator_fork(pkv_allocator* a, int64_t alloc_id, int32_t n_tokens, int64_t* new_id, int32_t* blocks,
                       int32_t capacity, int32_t* n_blocks) {
  if (!a || !new_id || n_tokens < 1) return PKV_EINVAL;
  auto it = a->allocs.find(alloc_id);
  if (it == a->allocs.end()) return PKV_EINVAL;
  const int32_t k = blocks_for(n_tokens, a->bs);
  if (k > (int32_t)it->second.blocks.size()) return PKV_EINVAL;
  if (blocks && capacity < k) return PKV_EINVAL;
  Allocation f{std::vector<int32_t>(it->second.blocks.begin(), it->second.blocks.begin() + k), it->second.node};
  for (int32_t b : f.blocks) a->holders[b] += 1;
  if (f.node != 0) a->nodes[f.node].refs += 1;
  const int64_t id = a->next_id++;
  const std::vector<int32_t> out = f.blocks;
  a->allocs[id] = std::move(f);
  *new_id = id;
  return copy_out(out, blocks, capacity, n_blocks);
}

int pkv_allocator_extend(pkv_allocator* a, int64_t alloc_id, int32_t n_total, int32_t* blocks, int32_t capacity,
                         int32_t* n_blocks) {
  if (!a || n_total < 1) return PKV_EINVAL;
  auto it = a->allocs.find(alloc_id);
  if (it == a->allocs.end()) return PKV_EINVAL;
  const int32_t k = blocks_for(n_total, a->bs);
  if (blocks && capacity < std::max<int32_t>(k, (int32_t)it->second.blocks.size())) return PKV_EINVAL;
  const int32_t extra = k - (int32_t)it->second.blocks.size();
  if (extra > 0) {
    a->clock += 1;
    if (!a->evict_until((size_t)extra)) return PKV_ENOSPACE;
    const std::vector<int32_t> fresh = a->take((size_t)extra);
    for (int32_t b : fresh) a->holders[b] += 1;
    it->second.blocks.insert(it->second.blocks.end(), fresh.begin(), fresh.end());
  }
  return copy_out(it->second.blocks, blocks, capacity, n_blocks);
}

int pkv_allocator_prepare_write(pkv_allocator* a, int64_t alloc_id, int32_t pos, int32_t* src, int32_t* dst) {
  if (!a || !src || !dst || pos < 0) return PKV_EINVAL;
  auto it = a->allocs.find(alloc_id);
  if (it == a->allocs.end()) return PKV_EINVAL;
  const int32_t i = pos / a->bs;
  if (i >= (int32_t)it->second.blocks.size()) return PKV_EINVAL;
  const int32_t b = it->second.blocks[i];
  *src = *dst = -1;
  if (a->holders[b] <= 1) return PKV_OK;
  a->clock += 1;
  if (!a->evict_until(1)) return PKV_ENOSPACE;
  const int32_t nb = a->take(1)[0];
  a->holders[nb] += 1;
  it->second.blocks[i] = nb;
  a->release(b);
  *src = b;
  *dst = nb;
  return PKV_OK;
}

int pkv_allocator_slots(pkv_allocator* a, int64_t alloc_id, int32_t start, int32_t count, int64_t* slots) {
  if (!a || start < 0 || count < 0 || (count > 0 && !slots)) return PKV_EINVAL;
  auto it = a->allocs.find(alloc_id);
  if (it == a->allocs.end()) return PKV_EINVAL;
  const std::vector<int32_t>& bl = it->second.blocks;
  if ((int64_t)start + count > (int64_t)bl.size() * a->bs) return PKV_EINVAL;
  for (int32_t p = 0; p < count; ++p) {
    const int32_t pos = start + p;
    slots[p] = (int64_t)bl[pos / a->bs] * a->bs + pos % a->bs;
  }
  return PKV_OK;
}

int pkv_allocator_table(pkv_allocator* a, int64_t alloc_id, int32_t* blocks, int32_t capacity, int32_t* n_blocks) {
  if (!a || !n_blocks) return PKV_EINVAL;
  auto it = a->allocs.find(alloc_id);
  if (it == a->allocs.end()) return PKV_EINVAL;
  return copy_out(it->second.blocks, blocks, capacity, n_blocks);
}

int32_t pkv_allocator_num_free(const pkv_allocator* a) { return a ? (int32_t)a->free_list.size() : -1; }

int32_t pkv_allocator_num_cached(const pkv_allocator* a) { return a ? a->cached_blocks() : -1; }

}  // extern "C"
