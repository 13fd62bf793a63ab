// Seeded scheduler walk over the host KV cache manager (msgl_kvcache.h),
// built with the address and undefined-behaviour sanitizers by
// tests/test_kvcache_sanitizers.py: continuous batching with prefix matching
// at admission, the prompt cached after prefill, one batched one-token
// allocation per decode step, pressure-driven release and eviction, caching
// on finish.  After every step it checks what the manager's model fixes:
// every page is free, evictable or protected (no page lost or doubled), each
// live row's table entries are slots of whole pages, and at the end nothing
// stays protected.  Prints "ok <counts>" and exits 0, or names the failed
// check and exits 1.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "msgl_kvcache.h"

namespace {

struct Running {
  std::vector<int32_t> ids;
  int64_t len;
  int64_t handle;
  int steps_left;
  int prompt;
};

int fail(const char* what, long long a, long long b) {
  std::printf("FAILED %s (%lld vs %lld)\n", what, a, b);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 7;
  const int32_t P = argc > 2 ? std::atoi(argv[2]) : 16;
  // a small pool, so that eviction, deferred admission and release happen
  const int64_t num_slots = argc > 3 ? std::atoll(argv[3]) : 8192;
  const int32_t max_rows = 24, max_len = 2048;
  std::mt19937_64 rng(seed);

  // 12 shared system prompts of 64-384 tokens, each request one of them plus
  // 16-160 own tokens, 4-40 decode steps
  std::vector<std::vector<int32_t>> systems(12);
  for (auto& s : systems) {
    s.resize(64 + rng() % 321);
    for (auto& t : s) t = (int32_t)(rng() % 32000);
  }
  const int num_requests = 300;
  std::vector<std::vector<int32_t>> prompts(num_requests);
  std::vector<int> steps(num_requests);
  for (int k = 0; k < num_requests; ++k) {
    prompts[k] = systems[rng() % systems.size()];
    const int own = 16 + (int)(rng() % 145);
    for (int i = 0; i < own; ++i) prompts[k].push_back((int32_t)(rng() % 32000));
    steps[k] = 4 + (int)(rng() % 37);
  }

  msgl_kv_cache* kv = nullptr;
  if (msgl_kvc_create(num_slots, P, max_rows, max_len, &kv) != MSGL_KVC_OK) return fail("create", 0, 0);
  const int64_t pages = num_slots / P;
  const int32_t* table = msgl_kvc_page_table(kv);

  std::vector<int> pending;
  for (int k = 0; k < num_requests; ++k) pending.push_back(k);
  std::map<int32_t, Running> running;
  long long admitted = 0, deferred = 0, decode_tokens = 0, evictions = 0, matched = 0;

  auto check = [&]() -> int {
    int64_t st[6];
    if (msgl_kvc_stats(kv, st, 6) != MSGL_KVC_OK) return fail("stats", 0, 0);
    // every page is free, or holds tree tokens, or holds a live row's own
    // (not yet cached) tokens; the tree holds whole pages
    int64_t own_pages = 0;
    for (const auto& [row, q] : running) {
      const int64_t n = msgl_kvc_row_len(kv, row);
      if (n < q.len) return fail("row shorter than its request", n, q.len);
      const int64_t cached = msgl_kvc_handle_len(kv, q.handle);
      if (cached < 0) return fail("locked handle not live", q.handle, 0);
      own_pages += (n + P - 1) / P - cached / P;
      for (int64_t j = 0; j < n; ++j) {
        const int32_t s = table[(int64_t)row * max_len + j];
        if (s < 0 || s >= pages * P) return fail("slot outside the pool", s, j);
        const int32_t first = table[(int64_t)row * max_len + (j - j % P)];
        if (s != first + (int32_t)(j % P)) return fail("page not contiguous", s, first);
      }
    }
    if ((st[1] + st[2]) % P != 0) return fail("tree tokens not whole pages", st[1] + st[2], P);
    const int64_t total = st[0] + (st[1] + st[2]) / P + own_pages;
    if (total != pages) return fail("pages not conserved", total, pages);
    return 0;
  };

  int guard = 0;
  bool throttled = false;   // after a release for lack of pages, admit nothing until a request ends
  while ((!pending.empty() || !running.empty()) && ++guard < 100000) {
    if (running.empty()) throttled = false;
    // admission
    while (!throttled && !pending.empty() && (int)running.size() < max_rows) {
      const int k = pending.front();
      const auto& ids = prompts[k];
      int32_t row = -1;
      if (msgl_kvc_alloc_row(kv, &row) != MSGL_KVC_OK) break;
      int64_t cl = 0, h = 0;
      if (msgl_kvc_match(kv, ids.data(), (int64_t)ids.size(), row, &cl, &h) != MSGL_KVC_OK)
        return fail("match", k, 0);
      if (msgl_kvc_lock(kv, h, 1) != MSGL_KVC_OK) return fail("lock", h, 0);
      const int64_t dev = (int64_t)ids.size();
      if (msgl_kvc_allocate(kv, 1, &row, &cl, &dev) != MSGL_KVC_OK) {
        if (msgl_kvc_release(kv, row, h) != MSGL_KVC_OK) return fail("release", row, h);
        if (msgl_kvc_free_row(kv, row) != MSGL_KVC_OK) return fail("free_row", row, 0);
        ++deferred;
        break;
      }
      int64_t h2 = 0, n2 = 0;
      if (msgl_kvc_cache_req(kv, row, ids.data(), dev, h, 0, &h2, &n2) != MSGL_KVC_OK)
        return fail("cache_req", row, 0);
      pending.erase(pending.begin());
      running[row] = Running{ids, dev, h2, steps[k], k};
      ++admitted;
      matched += cl;
    }
    if (int e = check()) return e;
    // one decode step for every running request
    if (!running.empty()) {
      std::vector<int32_t> rows;
      std::vector<int64_t> cur, next;
      for (const auto& [row, q] : running) {
        rows.push_back(row);
        cur.push_back(q.len);
        next.push_back(q.len + 1);
      }
      if (msgl_kvc_allocate(kv, (int32_t)rows.size(), rows.data(), cur.data(), next.data()) ==
          MSGL_KVC_OK) {
        for (auto& [row, q] : running) {
          q.ids.push_back((int32_t)(rng() % 32000));
          q.len += 1;
          q.steps_left -= 1;
        }
        decode_tokens += (long long)rows.size();
      } else {
        // out of pages: the newest request gives its pages back and waits
        const int32_t r = rows.back();
        Running q = running[r];
        running.erase(r);
        if (msgl_kvc_release(kv, r, q.handle) != MSGL_KVC_OK) return fail("release", r, 0);
        if (msgl_kvc_free_row(kv, r) != MSGL_KVC_OK) return fail("free_row", r, 0);
        pending.insert(pending.begin(), q.prompt);
        ++deferred;
        throttled = true;
      }
    }
    // finished requests are cached and their rows freed
    std::vector<int32_t> done;
    for (const auto& [row, q] : running)
      if (q.steps_left <= 0) done.push_back(row);
    for (int32_t r : done) {
      Running q = running[r];
      running.erase(r);
      int64_t h2 = 0, n2 = 0;
      if (msgl_kvc_cache_req(kv, r, q.ids.data(), q.len, q.handle, 1, &h2, &n2) != MSGL_KVC_OK)
        return fail("cache_req finished", r, 0);
      if (msgl_kvc_free_row(kv, r) != MSGL_KVC_OK) return fail("free_row", r, 0);
      throttled = false;
    }
    // now and then, evict a few pages ahead of need
    if (rng() % 8 == 0) {
      int64_t freed = 0;
      if (msgl_kvc_evict(kv, 1 + (int64_t)(rng() % 8), &freed) != MSGL_KVC_OK) return fail("evict", 0, 0);
      evictions += freed;
    }
    if (int e = check()) return e;
  }
  if (guard >= 100000) return fail("walk did not finish", guard, 0);

  int64_t st[6];
  msgl_kvc_stats(kv, st, 6);
  if (st[2] != 0) return fail("tokens still protected", st[2], 0);
  if (st[0] * P + st[1] != pages * P) return fail("free + evictable != pool", st[0] * P + st[1], pages * P);
  // evicting everything leaves the whole pool free and the tree empty
  int64_t freed = 0;
  msgl_kvc_evict(kv, pages, &freed);
  msgl_kvc_stats(kv, st, 6);
  if (st[0] != pages || st[3] != 0) return fail("full eviction", st[0], st[3]);
  msgl_kvc_destroy(kv);
  std::printf("ok admitted=%lld deferred=%lld decode_tokens=%lld matched=%lld evicted_pages=%lld\n",
              admitted, deferred, decode_tokens, matched, evictions + freed);
  return 0;
}
