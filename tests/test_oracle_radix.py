"""Pins of the KV cache manager oracle (page allocator + radix prefix cache) — CPU.

Each pin checks the oracle against something other than its own code:
* the worked example the pages draw (§4.4.4's tree: two prompts sharing a
  5-page run, one unrelated 2-page prompt) -> tests/golden/radix_tree_example.json;
* a flat brute-force model of prefix reuse: the longest page-aligned prefix of
  a query that any cached request shares, with the slots of the request that
  first cached it;
* conservation: every page is in exactly one of the free list, the tree, or a
  running request's own range;
* locking: protected + evictable = tokens in the tree, and eviction never
  touches a locked path;
* LRU: eviction takes the leaf whose last use is oldest (tracked by hand);
* the key compare against numpy.
Planted mistakes in a copy of the oracle's source must fail at least one pin.
"""

import json
import os
import types

import numpy as np
import pytest

import oracle
from oracle.radix import KVCacheOracle, compare_key, OK, ERR_FULL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "radix_tree_example.json")


def cache_prompt(kv, ids, finished=True):
    """Admit one request, compute its whole prompt, cache it (the scheduler
    path of §4.4.7).  Returns (row, handle, matched length)."""
    st, row = kv.alloc_row()
    assert st == OK
    st, cached, h = kv.match(ids, row)
    assert st == OK
    kv.lock(h, +1)
    assert kv.allocate([row], [cached], [len(ids)]) == OK
    st, nh, nl = kv.cache_req(row, ids, len(ids), h, finished)
    assert st == OK
    if finished:
        assert kv.free_row(row) == OK
    return row, nh, cached


def test_compare_key_matches_numpy():
    rng = np.random.default_rng(0)
    for _ in range(200):
        n = int(rng.integers(0, 20))
        a = rng.integers(0, 4, n)
        b = a.copy() if rng.random() < 0.5 else rng.integers(0, 4, int(rng.integers(0, 20)))
        m = min(len(a), len(b))
        ne = a[:m] != b[:m]
        want = int(np.argmax(ne)) if ne.any() else m
        assert compare_key(a, b) == want


def tree_shape(node, P):
    kids = sorted((tree_shape(c, P) for c in node.children.values()), key=json.dumps)
    return {"pages": len(node.key) // P, "children": kids}


def test_pages_example_tree():
    g = json.load(open(GOLDEN))
    P = g["page_size"]
    runs = {k: list(range(v["first_id"], v["first_id"] + v["pages"] * P)) for k, v in g["runs"].items()}
    kv = KVCacheOracle(1024, P, 8, 256)
    for req in g["requests"]:
        cache_prompt(kv, [t for run in req for t in runs[run]])
    got = sorted((tree_shape(c, P) for c in kv.root.children.values()), key=json.dumps)
    want = sorted(g["tree"]["children"], key=json.dumps)
    for w in want:
        w["children"] = sorted(w["children"], key=json.dumps)
    assert got == want
    # 5 + 3 + 3 + 2 pages are in the tree, the rest is free
    assert kv.stats()[0] == 1024 // P - 13 and kv.stats()[1] == 13 * P


def flat_match(cached, q, P):
    """Longest page-aligned prefix of q that some cached sequence shares, and
    the slots the first sequence to cache it holds there."""
    best, slots = 0, []
    for ids, sl in cached:
        k = compare_key(ids, q)
        k -= k % P
        if k > best:
            best, slots = k, list(sl[:k])
    return best, slots


@pytest.mark.parametrize("P", [1, 4, 16])
def test_match_equals_flat_longest_prefix(P):
    rng = np.random.default_rng(P)
    kv = KVCacheOracle(1 << 14, P, 16, 512)
    stems = [list(rng.integers(0, 50, int(rng.integers(P, 6 * P)))) for _ in range(6)]
    cached = []          # (ids, slots) in insertion order; the tree keeps the first slots
    for it in range(60):
        ids = list(stems[int(rng.integers(0, 6))]) + list(rng.integers(0, 50, int(rng.integers(0, 4 * P))))
        ids = ids[:int(rng.integers(1, len(ids) + 1))]
        st, row = kv.alloc_row()
        st, cached_len, h = kv.match(ids, row)
        want_len, want_slots = flat_match(cached, ids, P)
        assert cached_len == want_len, it
        assert list(kv.table[row, :cached_len]) == want_slots
        kv.lock(h, +1)
        assert kv.allocate([row], [cached_len], [len(ids)]) == OK
        n_al = len(ids) - len(ids) % P
        slots = list(kv.table[row, :n_al])
        kv.cache_req(row, ids, len(ids), h, True)
        kv.free_row(row)
        if n_al:
            # the tree now holds ids[:n_al]; a prefix it already had keeps its slots
            prev_len, prev_slots = flat_match(cached, ids[:n_al], P)
            cached.append((ids[:n_al], prev_slots + slots[prev_len:]))


def owned_pages(kv, running):
    out = []
    for row, h in running.items():
        for j in range(h.depth, kv.row_len[row], kv.P):
            out.append(int(kv.table[row, j]))
    return out


def tree_pages(kv):
    out, stack = [], [kv.root]
    while stack:
        nd = stack.pop()
        for ch in nd.children.values():
            out.extend(int(s) for s in ch.value[::kv.P])
            stack.append(ch)
    return out


def check_invariants(kv, running, num_pages):
    pages = list(kv.free_pages) + tree_pages(kv) + owned_pages(kv, running)
    assert sorted(pages) == [p * kv.P for p in range(num_pages)], "pages lost or doubly owned"
    tree_tokens = sum(len(nd.key) for ids, nd in _nodes(kv))
    assert kv.evictable + kv.protected == tree_tokens
    assert kv.protected == sum(len(nd.key) for _, nd in _nodes(kv) if nd.ref > 0)


def _nodes(kv):
    out, stack = [], [kv.root]
    while stack:
        nd = stack.pop()
        for ch in nd.children.values():
            out.append((None, ch))
            stack.append(ch)
    return out


@pytest.mark.parametrize("P", [1, 8])
def test_conservation_and_locking_under_a_scheduler_walk(P):
    rng = np.random.default_rng(10 + P)
    num_pages = 96
    kv = KVCacheOracle(num_pages * P, P, 12, 64 * P)
    stems = [list(rng.integers(0, 30, int(rng.integers(2 * P, 8 * P)))) for _ in range(4)]
    running = {}        # row -> handle
    lens, ids_of = {}, {}
    for it in range(400):
        op = rng.random()
        if op < 0.35 and kv.free_rows:
            ids = stems[int(rng.integers(0, 4))] + list(rng.integers(0, 30, int(rng.integers(1, 6 * P))))
            st, row = kv.alloc_row()
            st, cl, h = kv.match(ids, row)
            kv.lock(h, +1)
            if kv.allocate([row], [cl], [len(ids)]) != OK:
                kv.release(row, h)
                kv.free_row(row)
            else:
                st, h2, _ = kv.cache_req(row, ids, len(ids), h, False)
                running[row], lens[row], ids_of[row] = h2, len(ids), ids
        elif op < 0.75 and running:
            row = list(running)[int(rng.integers(0, len(running)))]
            if lens[row] + 1 <= kv.max_len and kv.allocate([row], [lens[row]], [lens[row] + 1]) == OK:
                ids_of[row] = ids_of[row] + [int(rng.integers(0, 30))]
                lens[row] += 1
        elif running:
            row = list(running)[int(rng.integers(0, len(running)))]
            if rng.random() < 0.7:
                kv.cache_req(row, ids_of[row], lens[row], running[row], True)
            else:
                kv.release(row, running[row])
            del running[row]
            kv.free_row(row)
        check_invariants(kv, running, num_pages)
        # a locked path survives any eviction
        if it % 50 == 49:
            before = {id(nd) for _, nd in _nodes(kv) if nd.ref > 0}
            kv.evict(10 ** 6)
            after = {id(nd) for _, nd in _nodes(kv)}
            assert before <= after
            assert kv.evictable == 0
            check_invariants(kv, running, num_pages)


def test_eviction_is_least_recently_used_first():
    P = 2
    kv = KVCacheOracle(256, P, 8, 64)
    seqs = [[100 * k + i for i in range(4 * P)] for k in range(5)]
    last_use = {}
    for k, s in enumerate(seqs):
        cache_prompt(kv, s)
        last_use[k] = kv.clock
    # touch 3, 0 and 4 again (match refreshes the nodes it walks)
    for k in (3, 0, 4):
        kv.match(seqs[k])
        last_use[k] = kv.clock
    order = []
    while kv.stats()[1] > 0:
        before = {tuple(ids) for ids, _ in kv.sequences()}
        kv.evict(1)
        after = {tuple(ids) for ids, _ in kv.sequences()}
        gone = [k for k, s in enumerate(seqs) if tuple(s) in before and tuple(s) not in after]
        order += gone
    assert order == sorted(last_use, key=lambda k: last_use[k])


def test_concurrent_prompts_are_deduplicated_on_caching():
    P = 4
    kv = KVCacheOracle(512, P, 8, 128)
    ids = list(range(1, 30))
    rows, hs = [], []
    for _ in range(2):                       # both admitted before either is cached
        st, row = kv.alloc_row()
        st, cl, h = kv.match(ids, row)
        assert cl == 0
        kv.lock(h, +1)
        assert kv.allocate([row], [0], [len(ids)]) == OK
        rows.append(row)
        hs.append(h)
    free0 = kv.stats()[0]
    st, h0, l0 = kv.cache_req(rows[0], ids, len(ids), hs[0], False)
    st, h1, l1 = kv.cache_req(rows[1], ids, len(ids), hs[1], False)
    assert l0 == l1 == 28 and h0 is h1
    # the second request's 7 duplicate pages went back; its row now reads the first's
    assert kv.stats()[0] == free0 + 7
    assert np.array_equal(kv.table[rows[1], :28], kv.table[rows[0], :28])
    assert kv.table[rows[1], 28] != kv.table[rows[0], 28]      # own partial page kept


def test_full_pool_reports_full_after_evicting_what_it_can():
    P = 4
    kv = KVCacheOracle(16 * P, P, 4, 64)
    st, row = kv.alloc_row()
    kv.allocate([row], [0], [10 * P])
    kv.cache_req(row, list(range(10 * P)), 10 * P, kv.root, False)   # 10 pages locked
    st, r2 = kv.alloc_row()
    assert kv.allocate([r2], [0], [7 * P]) == ERR_FULL                 # 6 free, nothing evictable
    assert kv.allocate([r2], [0], [6 * P - 3]) == OK                   # 6 pages, the last in part
    assert kv.stats()[0] == 0
    # decode steps inside r2's last page need no new page, even with none free
    for n in range(6 * P - 3, 6 * P):
        assert kv.allocate([r2], [n], [n + 1]) == OK
    assert kv.allocate([r2], [6 * P], [6 * P + 1]) == ERR_FULL


MUTANTS = [
    ("m -= m % self.P                       # only whole pages match", "pass"),
    ("node = self._split(child, m)\n                break", "node = child\n                break"),
    ("key=lambda x: (x.stamp, x.serial)", "key=lambda x: (-x.stamp, x.serial)"),
    ("self.evictable -= delta * len(node.key)\n                self.protected += delta * len(node.key)",
     "self.evictable += delta * len(node.key)\n                self.protected -= delta * len(node.key)"),
    ("if not ch.children and ch.ref == 0:", "if not ch.children:"),
    ("            self._free_run(t, old.depth, matched)\n", ""),
    ("        if matched > old.depth:", "        if False:"),
    ("node.stamp = self.clock", "pass"),
    ("total += up(d) // P - up(c) // P", "total += up(d) // P - c // P"),
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistakes_are_caught(old, new):
    import oracle.radix as mod0
    src = open(mod0.__file__).read()
    assert old in src
    mod = types.ModuleType("radix_mutant")
    exec(compile(src.replace(old, new, 1), "radix_mutant", "exec"), mod.__dict__)
    g = globals()
    saved = g["KVCacheOracle"]
    g["KVCacheOracle"] = mod.KVCacheOracle
    failed = 0
    try:
        for pin in (test_pages_example_tree, lambda: test_match_equals_flat_longest_prefix(4),
                    lambda: test_conservation_and_locking_under_a_scheduler_walk(8),
                    test_eviction_is_least_recently_used_first,
                    test_concurrent_prompts_are_deduplicated_on_caching,
                    test_full_pool_reports_full_after_evicting_what_it_can):
            try:
                pin()
            except Exception:
                failed += 1
    finally:
        g["KVCacheOracle"] = saved
    assert failed > 0
