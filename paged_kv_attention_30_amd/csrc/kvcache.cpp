// Host-side KV cache manager: page allocator + radix prefix cache.
//
// "Mini-SGLang complete analysis" §4.4 (KV cache pool and radix prefix cache):
//   §4.4.2 three layers: a cache manager (free slots, prefix cache, page
//          table) above a prefix cache and the KV pool;
//   §4.4.4 the radix tree: every node is an edge holding a run of token ids
//          and the pool slots of their K/V, a reference count (0 = evictable)
//          and an LRU timestamp; the root is never evicted;
//   §4.4.5 prefix matching walks the children keyed by the first page of
//          token ids, compares a node's edge with the query (first
//          mismatch), rounds the match down to whole pages and splits a node
//          that matches only in part;
//   §4.4.6 locking adds +-1 along the path to the root and moves sizes
//          between evictable and protected; eviction pops unlocked leaves
//          oldest first and lets a parent that becomes an unlocked leaf join
//          the candidates;
//   §4.4.7 allocation gives every request ceil(device_len / P) -
//          ceil(cached_len / P) new pages (evicting first when short) and
//          writes them into its page-table row; caching a request inserts its
//          computed prefix, frees the pages that duplicate what the tree
//          already held, and either keeps the new path locked or (finished)
//          frees the unaligned tail.
// "Mini-sglang deep-analysis report" (KV cache management): the protected /
// evictable / free split of the pool, lazy eviction of unlocked leaves.
//
// Readings where the pages are silent or garbled:
//   * the free list holds one entry per page (its first slot) and is a FIFO:
//     allocation takes from the front, frees and evictions append;
//   * timestamps come from a logical clock (one tick per match / insert), and
//     ties between leaves are broken by node creation order, so eviction
//     order is reproducible;
//   * locking moves a node's tokens from evictable to protected (the printed
//     sign of that update is inverted in the page; its comment and the rest
//     of the section fix the direction);
//   * eviction is asked for pages and frees whole nodes until at least that
//     many pages are free;
//   * when caching finds part of the request's prefix already in the tree
//     (another request inserted it first), the request's own pages there are
//     freed and its page-table row is pointed at the tree's pages, which hold
//     the same K/V.
//
// Not thread-safe: one manager serves one scheduler thread.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

#include "msgl_kvcache.h"

namespace {

// Exact key of a child: the first page of its token ids.
struct PageKey {
  std::vector<int32_t> ids;
  bool operator==(const PageKey& o) const { return ids == o.ids; }
};
struct PageKeyHash {
  size_t operator()(const PageKey& k) const {
    uint64_t h = 1469598103934665603ull;
    for (int32_t v : k.ids) {
      h ^= (uint32_t)v;
      h *= 1099511628211ull;
    }
    return (size_t)h;
  }
};

struct Node {
  int64_t parent = -1;
  std::vector<int32_t> key;     // token ids of this edge
  std::vector<int32_t> value;   // their pool slots
  std::unordered_map<PageKey, int64_t, PageKeyHash> children;
  int64_t depth = 0;            // tokens from the root to the end of this edge
  int64_t ref = 0;
  uint64_t stamp = 0;
  uint64_t serial = 0;          // creation order (LRU tie-break)
  bool alive = false;
};

}  // namespace

struct msgl_kv_cache {
  int64_t num_slots = 0;
  int32_t page = 1;
  int32_t max_rows = 0;
  int32_t max_len = 0;
  std::vector<Node> nodes;              // node 0 is the root
  std::vector<int64_t> free_nodes;
  std::deque<int32_t> free_pages;       // first slot of each free page
  std::vector<int32_t> table;           // [max_rows, max_len]
  std::vector<int64_t> row_len;         // slots a row owns through [0, row_len)
  std::vector<uint8_t> row_used;
  std::deque<int32_t> free_rows;
  int64_t evictable = 0;                // tokens in unlocked nodes
  int64_t protected_ = 0;               // tokens in locked nodes
  uint64_t clock = 0;
  uint64_t serial = 0;
};

namespace {

PageKey first_page(const int32_t* ids, int32_t page) {
  return PageKey{std::vector<int32_t>(ids, ids + page)};
}

int64_t new_node(msgl_kv_cache* c) {
  int64_t id;
  if (!c->free_nodes.empty()) {
    id = c->free_nodes.back();
    c->free_nodes.pop_back();
    c->nodes[id] = Node();
  } else {
    id = (int64_t)c->nodes.size();
    c->nodes.emplace_back();
  }
  c->nodes[id].alive = true;
  c->nodes[id].serial = ++c->serial;
  return id;
}

bool valid_handle(const msgl_kv_cache* c, int64_t h) {
  return h >= 0 && h < (int64_t)c->nodes.size() && c->nodes[h].alive;
}

int64_t align_down(int64_t x, int32_t p) { return x - x % p; }
int64_t align_up(int64_t x, int32_t p) { return (x + p - 1) / p * p; }

// Split node `n` after its first `m` tokens (0 < m < length, m a whole
// number of pages): a new parent takes [0, m) and inherits the count and
// timestamp; `n` keeps [m, length).  Returns the new parent.
int64_t split_at(msgl_kv_cache* c, int64_t n, int64_t m) {
  const int64_t p = new_node(c);
  Node& par = c->nodes[p];
  Node& nd = c->nodes[n];
  par.parent = nd.parent;
  par.key.assign(nd.key.begin(), nd.key.begin() + m);
  par.value.assign(nd.value.begin(), nd.value.begin() + m);
  par.depth = nd.depth - (int64_t)nd.key.size() + m;
  par.ref = nd.ref;
  par.stamp = nd.stamp;
  const PageKey k = first_page(nd.key.data(), c->page);
  c->nodes[nd.parent].children[k] = p;
  nd.key.erase(nd.key.begin(), nd.key.begin() + m);
  nd.value.erase(nd.value.begin(), nd.value.begin() + m);
  nd.parent = p;
  par.children[first_page(nd.key.data(), c->page)] = n;
  return p;
}

// Longest page-aligned prefix of ids[0, n) held by the tree.  Nodes matched
// in full are touched; a node matched in part is split and its new parent is
// the result.
int64_t walk(msgl_kv_cache* c, const int32_t* ids, int64_t n, int64_t* prefix_out) {
  const uint64_t tic = ++c->clock;
  int64_t node = 0;
  int64_t prefix = 0;
  while (n - prefix >= c->page) {
    auto it = c->nodes[node].children.find(first_page(ids + prefix, c->page));
    if (it == c->nodes[node].children.end()) break;
    const int64_t child = it->second;
    const std::vector<int32_t>& key = c->nodes[child].key;
    const int64_t len = std::min<int64_t>((int64_t)key.size(), n - prefix);
    const int64_t m0 = std::mismatch(key.begin(), key.begin() + len, ids + prefix).first - key.begin();
    const int64_t m = align_down(m0, c->page);
    prefix += m;
    if (m != (int64_t)key.size()) {
      node = split_at(c, child, m);
      break;
    }
    node = child;
    c->nodes[node].stamp = tic;
  }
  *prefix_out = prefix;
  return node;
}

// slots of the path root -> node, in token order
void path_slots(const msgl_kv_cache* c, int64_t node, int32_t* out) {
  while (node != 0) {
    const Node& nd = c->nodes[node];
    const int64_t start = nd.depth - (int64_t)nd.value.size();
    std::copy(nd.value.begin(), nd.value.end(), out + start);
    node = nd.parent;
  }
}

void lock_path(msgl_kv_cache* c, int64_t node, int delta) {
  while (node != 0) {
    Node& nd = c->nodes[node];
    const bool was_zero = nd.ref == 0;
    nd.ref += delta;
    const bool now_zero = nd.ref == 0;
    if (was_zero != now_zero) {
      const int64_t len = (int64_t)nd.key.size();
      c->evictable -= delta * len;
      c->protected_ += delta * len;
    }
    node = nd.parent;
  }
}

// Return the pages of slots[lo, hi) (lo page-aligned) to the free list.
void free_run(msgl_kv_cache* c, const int32_t* slots, int64_t lo, int64_t hi) {
  for (int64_t j = lo; j < hi; j += c->page) c->free_pages.push_back(slots[j]);
}

// Evict unlocked leaves, oldest first, until `pages` pages were freed or
// nothing is left to evict.  Returns the pages freed.
int64_t evict_pages(msgl_kv_cache* c, int64_t pages) {
  using Item = std::pair<std::pair<uint64_t, uint64_t>, int64_t>;   // ((stamp, serial), node)
  std::priority_queue<Item, std::vector<Item>, std::greater<Item>> heap;
  for (int64_t i = 1; i < (int64_t)c->nodes.size(); ++i) {
    const Node& nd = c->nodes[i];
    if (nd.alive && nd.children.empty() && nd.ref == 0)
      heap.push({{nd.stamp, nd.serial}, i});
  }
  int64_t freed = 0;
  while (freed < pages && !heap.empty()) {
    const int64_t n = heap.top().second;
    heap.pop();
    Node& nd = c->nodes[n];
    const int64_t len = (int64_t)nd.value.size();
    free_run(c, nd.value.data(), 0, len);
    freed += len / c->page;
    c->evictable -= len;
    const int64_t par = nd.parent;
    c->nodes[par].children.erase(first_page(nd.key.data(), c->page));
    nd = Node();
    c->free_nodes.push_back(n);
    const Node& pn = c->nodes[par];
    if (par != 0 && pn.children.empty() && pn.ref == 0) heap.push({{pn.stamp, pn.serial}, par});
  }
  return freed;
}

bool row_ok(const msgl_kv_cache* c, int32_t row) {
  return row >= 0 && row < c->max_rows && c->row_used[row];
}

}  // namespace

extern "C" {

int msgl_kvc_create(int64_t num_slots, int32_t page_size, int32_t max_rows, int32_t max_len,
                    msgl_kv_cache** out) {
  if (!out) return MSGL_KVC_ERR_ARG;
  *out = nullptr;
  if (page_size < 1 || num_slots < page_size || num_slots > INT32_MAX || max_rows < 1 ||
      max_len < 1 || max_len % page_size != 0)
    return MSGL_KVC_ERR_ARG;
  msgl_kv_cache* c = new (std::nothrow) msgl_kv_cache();
  if (!c) return MSGL_KVC_ERR_NOMEM;
  try {
    c->num_slots = num_slots;
    c->page = page_size;
    c->max_rows = max_rows;
    c->max_len = max_len;
    c->nodes.emplace_back();
    c->nodes[0].alive = true;
    c->nodes[0].ref = 1;   // the root is never evicted
    for (int64_t s = 0; s + page_size <= num_slots; s += page_size) c->free_pages.push_back((int32_t)s);
    c->table.assign((size_t)max_rows * max_len, 0);
    c->row_len.assign(max_rows, 0);
    c->row_used.assign(max_rows, 0);
    for (int32_t r = 0; r < max_rows; ++r) c->free_rows.push_back(r);
  } catch (...) {
    delete c;
    return MSGL_KVC_ERR_NOMEM;
  }
  *out = c;
  return MSGL_KVC_OK;
}

void msgl_kvc_destroy(msgl_kv_cache* c) { delete c; }

const int32_t* msgl_kvc_page_table(const msgl_kv_cache* c) { return c ? c->table.data() : nullptr; }

int msgl_kvc_alloc_row(msgl_kv_cache* c, int32_t* row) {
  if (!c || !row) return MSGL_KVC_ERR_ARG;
  if (c->free_rows.empty()) return MSGL_KVC_ERR_FULL;
  *row = c->free_rows.front();
  c->free_rows.pop_front();
  c->row_used[*row] = 1;
  c->row_len[*row] = 0;
  return MSGL_KVC_OK;
}

int msgl_kvc_free_row(msgl_kv_cache* c, int32_t row) {
  if (!c || !row_ok(c, row)) return MSGL_KVC_ERR_ARG;
  if (c->row_len[row] != 0) return MSGL_KVC_ERR_STATE;   // release its pages first
  c->row_used[row] = 0;
  c->free_rows.push_back(row);
  return MSGL_KVC_OK;
}

int msgl_kvc_match(msgl_kv_cache* c, const int32_t* ids, int64_t n, int32_t row,
                   int64_t* cached_len, int64_t* handle) {
  if (!c || (n > 0 && !ids) || n < 0 || !cached_len || !handle) return MSGL_KVC_ERR_ARG;
  if (row >= 0 && (!row_ok(c, row) || c->row_len[row] != 0 || n > c->max_len))
    return MSGL_KVC_ERR_ARG;
  try {
    int64_t prefix = 0;
    const int64_t node = walk(c, ids, n, &prefix);
    if (row >= 0) path_slots(c, node, c->table.data() + (size_t)row * c->max_len);
    *cached_len = prefix;
    *handle = node;
  } catch (...) {
    return MSGL_KVC_ERR_NOMEM;
  }
  return MSGL_KVC_OK;
}

int msgl_kvc_lock(msgl_kv_cache* c, int64_t handle, int32_t delta) {
  if (!c || !valid_handle(c, handle) || (delta != 1 && delta != -1)) return MSGL_KVC_ERR_ARG;
  if (delta < 0) {
    for (int64_t n = handle; n != 0; n = c->nodes[n].parent)
      if (c->nodes[n].ref <= 0) return MSGL_KVC_ERR_STATE;   // unlock of an unlocked path
  }
  lock_path(c, handle, delta);
  return MSGL_KVC_OK;
}

int msgl_kvc_allocate(msgl_kv_cache* c, int32_t n, const int32_t* rows, const int64_t* cached_lens,
                      const int64_t* device_lens) {
  if (!c || n < 0 || (n > 0 && (!rows || !cached_lens || !device_lens))) return MSGL_KVC_ERR_ARG;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t r = rows[i];
    if (!row_ok(c, r) || cached_lens[i] < 0 || device_lens[i] < cached_lens[i] ||
        device_lens[i] > c->max_len)
      return MSGL_KVC_ERR_ARG;
    // pages past the cached tokens are new: the row may not own any there
    if (c->row_len[r] > align_up(cached_lens[i], c->page)) return MSGL_KVC_ERR_STATE;
    total += align_up(device_lens[i], c->page) / c->page - align_up(cached_lens[i], c->page) / c->page;
  }
  try {
    if (total > (int64_t)c->free_pages.size()) evict_pages(c, total - (int64_t)c->free_pages.size());
  } catch (...) {
    return MSGL_KVC_ERR_NOMEM;
  }
  if (total > (int64_t)c->free_pages.size()) return MSGL_KVC_ERR_FULL;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t r = rows[i];
    int32_t* t = c->table.data() + (size_t)r * c->max_len;
    const int64_t lo = align_up(cached_lens[i], c->page);
    const int64_t hi = align_up(device_lens[i], c->page);
    for (int64_t j = lo; j < hi; j += c->page) {
      const int32_t s = c->free_pages.front();
      c->free_pages.pop_front();
      for (int32_t e = 0; e < c->page; ++e) t[j + e] = s + e;
    }
    c->row_len[r] = std::max(c->row_len[r], hi);
  }
  return MSGL_KVC_OK;
}

int msgl_kvc_cache_req(msgl_kv_cache* c, int32_t row, const int32_t* ids, int64_t cached_len,
                       int64_t old_handle, int32_t finished, int64_t* new_handle,
                       int64_t* new_len) {
  if (!c || !row_ok(c, row) || (cached_len > 0 && !ids) || cached_len < 0 ||
      cached_len > c->row_len[row] || !valid_handle(c, old_handle) || !new_handle || !new_len)
    return MSGL_KVC_ERR_ARG;
  const int64_t old_len = c->nodes[old_handle].depth;
  if (old_len > cached_len) return MSGL_KVC_ERR_ARG;
  try {
    int32_t* t = c->table.data() + (size_t)row * c->max_len;
    const int64_t n_al = align_down(cached_len, c->page);
    int64_t matched = 0;
    int64_t node = walk(c, ids, n_al, &matched);
    if (matched < n_al) {
      const int64_t leaf = new_node(c);
      Node& lf = c->nodes[leaf];
      lf.parent = node;
      lf.key.assign(ids + matched, ids + n_al);
      lf.value.assign(t + matched, t + n_al);
      lf.depth = n_al;
      lf.stamp = c->clock;
      c->nodes[node].children[first_page(ids + matched, c->page)] = leaf;
      c->evictable += n_al - matched;
      node = leaf;
    }
    lock_path(c, old_handle, -1);
    if (matched > old_len) {
      // another request put [old_len, matched) into the tree first: free our
      // copies and point the row at the tree's pages (the same K/V)
      free_run(c, t, old_len, matched);
      std::vector<int32_t> path((size_t)n_al);
      path_slots(c, node, path.data());
      std::copy(path.begin() + old_len, path.begin() + matched, t + old_len);
    }
    if (finished) {
      free_run(c, t, n_al, c->row_len[row]);
      c->row_len[row] = 0;
    } else {
      lock_path(c, node, +1);
    }
    *new_handle = node;
    *new_len = n_al;
  } catch (...) {
    return MSGL_KVC_ERR_NOMEM;
  }
  return MSGL_KVC_OK;
}

int msgl_kvc_release(msgl_kv_cache* c, int32_t row, int64_t handle) {
  if (!c || !row_ok(c, row) || !valid_handle(c, handle)) return MSGL_KVC_ERR_ARG;
  const int64_t len = c->nodes[handle].depth;
  const int rc = msgl_kvc_lock(c, handle, -1);
  if (rc != MSGL_KVC_OK) return rc;
  free_run(c, c->table.data() + (size_t)row * c->max_len, len, c->row_len[row]);
  c->row_len[row] = 0;
  return MSGL_KVC_OK;
}

int msgl_kvc_evict(msgl_kv_cache* c, int64_t pages, int64_t* freed) {
  if (!c || pages < 0) return MSGL_KVC_ERR_ARG;
  try {
    const int64_t f = evict_pages(c, pages);
    if (freed) *freed = f;
  } catch (...) {
    return MSGL_KVC_ERR_NOMEM;
  }
  return MSGL_KVC_OK;
}

int msgl_kvc_stats(const msgl_kv_cache* c, int64_t* out, int32_t n) {
  if (!c || !out || n < 1) return MSGL_KVC_ERR_ARG;
  int64_t nodes = 0;
  for (const Node& nd : c->nodes) nodes += nd.alive ? 1 : 0;
  const int64_t v[6] = {(int64_t)c->free_pages.size(), c->evictable, c->protected_, nodes - 1,
                        (int64_t)c->free_rows.size(), (int64_t)c->clock};
  for (int32_t i = 0; i < n && i < 6; ++i) out[i] = v[i];
  return MSGL_KVC_OK;
}

int64_t msgl_kvc_free_list(const msgl_kv_cache* c, int32_t* out, int64_t cap) {
  if (!c) return -1;
  const int64_t n = (int64_t)c->free_pages.size();
  if (out) std::copy_n(c->free_pages.begin(), std::min(n, cap), out);
  return n;
}

int64_t msgl_kvc_row_len(const msgl_kv_cache* c, int32_t row) {
  if (!c || !row_ok(c, row)) return -1;
  return c->row_len[row];
}

int64_t msgl_kvc_handle_len(const msgl_kv_cache* c, int64_t handle) {
  if (!c || !valid_handle(c, handle)) return -1;
  return c->nodes[handle].depth;
}

int64_t msgl_compare_key(const int32_t* a, int64_t na, const int32_t* b, int64_t nb) {
  const int64_t n = std::min(na, nb);
  if (n <= 0) return 0;
  return std::mismatch(a, a + n, b).first - a;
}

}  // extern "C"
