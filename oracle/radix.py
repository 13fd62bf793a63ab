"""Plain CPU oracle for the host-side KV cache manager: page allocator + radix
prefix cache.

TEST INFRASTRUCTURE ONLY — see ``oracle/__init__.py``.  Nothing in the
library imports this module; it imports nothing from the library.

Source: "Mini-SGLang complete analysis" (blog.rzhang-lab.cn), §4.4:
  - §4.4.4: a radix tree whose nodes are edges, each holding a run of token
    ids, the pool slots of their K/V, a reference count (0 means the node may
    be evicted) and a last-use time; the root is created locked and is never
    evicted;
  - §4.4.5: matching walks the children keyed by the first page of ids,
    counts the common prefix of the node's run and the query (first
    mismatch), rounds it down to whole pages, and splits a node matched only
    in part into a new parent (the matched part, inheriting count and time)
    and itself (the rest); nodes matched in full get the walk's time;
  - §4.4.6: locking walks to the root adding +-1 and moves a node's size
    between "evictable" and "protected" when its count crosses zero;
    eviction pops unlocked leaves oldest first, and a parent left as an
    unlocked leaf becomes a candidate;
  - §4.4.7: allocate_paged gives each request ceil(device/P) - ceil(cached/P)
    new pages, evicting first when the free list is short, and writes them to
    its page-table row; cache_req inserts the computed prefix, unlocks the old
    handle, frees the pages the tree already held, and either locks the new
    handle or (finished) frees the tail.
"Mini-sglang deep-analysis report" (nightvoyager.top), KV cache management:
protected / evictable / free.

Readings where the pages are silent or garbled:
  * the free list holds whole pages (the first slot of each) in FIFO order;
  * time is a logical clock, one tick per walk; leaves with equal times are
    evicted in node creation order;
  * locking moves size from evictable to protected (the printed update has
    the opposite sign; the comment beside it and the section fix the
    direction);
  * eviction is asked for pages;
  * pages of a request that the tree already held when it is cached are freed
    and the request's row is pointed at the tree's pages.
"""

from __future__ import annotations

from collections import deque

import numpy as np

OK, ERR_ARG, ERR_FULL, ERR_STATE = 0, -1, -2, -3


def compare_key(a, b) -> int:
    """Length of the common prefix of two id sequences (the first position
    where they differ).  [§4.4.5, the key compare]"""
    n = min(len(a), len(b))
    i = 0
    while i < n and int(a[i]) == int(b[i]):
        i += 1
    return i


class Node:
    def __init__(self, serial: int):
        self.parent: Node | None = None
        self.key: list[int] = []
        self.value: list[int] = []
        self.children: dict[tuple, Node] = {}
        self.depth = 0
        self.ref = 0
        self.stamp = 0
        self.serial = serial
        self.alive = True


class KVCacheOracle:
    """The manager of §4.4.7 over the tree of §4.4.4-4.4.6."""

    def __init__(self, num_slots: int, page_size: int, max_rows: int, max_len: int):
        self.P = page_size
        self.max_rows = max_rows
        self.max_len = max_len
        self.serial = 0
        self.clock = 0
        self.root = self._new_node()
        self.root.ref = 1                       # the root is never evicted
        self.free_pages = deque(range(0, num_slots - page_size + 1, page_size))
        self.table = np.zeros((max_rows, max_len), dtype=np.int32)
        self.row_len = [0] * max_rows
        self.row_used = [False] * max_rows
        self.free_rows = deque(range(max_rows))
        self.evictable = 0
        self.protected = 0

    # -- tree ---------------------------------------------------------------
    def _new_node(self) -> Node:
        self.serial += 1
        return Node(self.serial)

    def _page_key(self, ids, start: int) -> tuple:
        return tuple(int(x) for x in ids[start:start + self.P])

    def _split(self, node: Node, m: int) -> Node:
        """[§4.4.5 split_at] node keeps [m:], a new parent takes [:m]."""
        par = self._new_node()
        par.parent = node.parent
        par.key = node.key[:m]
        par.value = node.value[:m]
        par.depth = node.depth - len(node.key) + m
        par.ref = node.ref
        par.stamp = node.stamp
        node.parent.children[tuple(node.key[:self.P])] = par
        node.key = node.key[m:]
        node.value = node.value[m:]
        node.parent = par
        par.children[tuple(node.key[:self.P])] = node
        return par

    def _walk(self, ids, n: int):
        """[§4.4.5 tree walk] -> (node, page-aligned prefix length)."""
        self.clock += 1
        node, prefix = self.root, 0
        while n - prefix >= self.P:
            child = node.children.get(self._page_key(ids, prefix))
            if child is None:
                break
            upto = min(len(child.key), n - prefix)
            m = compare_key(child.key[:upto], ids[prefix:prefix + upto])
            m -= m % self.P                       # only whole pages match
            prefix += m
            if m != len(child.key):
                node = self._split(child, m)
                break
            node = child
            node.stamp = self.clock
        return node, prefix

    def _path(self, node: Node) -> list[int]:
        runs = []
        while node is not self.root:
            runs.append(node.value)
            node = node.parent
        return [s for run in reversed(runs) for s in run]

    def _lock(self, node: Node, delta: int):
        """[§4.4.6 lock_handle]"""
        while node is not self.root:
            was_zero = node.ref == 0
            node.ref += delta
            if was_zero != (node.ref == 0):
                self.evictable -= delta * len(node.key)
                self.protected += delta * len(node.key)
            node = node.parent

    def _free_run(self, slots, lo: int, hi: int):
        for j in range(lo, hi, self.P):
            self.free_pages.append(int(slots[j]))

    def _leaves(self):
        out, stack = [], [self.root]
        while stack:
            nd = stack.pop()
            for ch in nd.children.values():
                stack.append(ch)
                if not ch.children and ch.ref == 0:
                    out.append(ch)
        return out

    def _evict(self, pages: int) -> int:
        """[§4.4.6 evict] unlocked leaves, oldest first."""
        cand = self._leaves()
        freed = 0
        while freed < pages and cand:
            node = min(cand, key=lambda x: (x.stamp, x.serial))
            cand.remove(node)
            self._free_run(node.value, 0, len(node.value))
            freed += len(node.value) // self.P
            self.evictable -= len(node.value)
            par = node.parent
            del par.children[tuple(node.key[:self.P])]
            node.alive = False
            if par is not self.root and not par.children and par.ref == 0:
                cand.append(par)
        return freed

    # -- manager (§4.4.7) ---------------------------------------------------
    def alloc_row(self):
        if not self.free_rows:
            return ERR_FULL, None
        r = self.free_rows.popleft()
        self.row_used[r] = True
        self.row_len[r] = 0
        return OK, r

    def free_row(self, row: int) -> int:
        if not (0 <= row < self.max_rows and self.row_used[row]):
            return ERR_ARG
        if self.row_len[row] != 0:
            return ERR_STATE
        self.row_used[row] = False
        self.free_rows.append(row)
        return OK

    def match(self, ids, row: int = -1):
        """match_req: (status, cached_len, handle node)."""
        if row >= 0 and (not self.row_used[row] or self.row_len[row] != 0 or len(ids) > self.max_len):
            return ERR_ARG, 0, None
        node, prefix = self._walk(ids, len(ids))
        if row >= 0:
            self.table[row, :prefix] = self._path(node)
        return OK, prefix, node

    def lock(self, node: Node, delta: int) -> int:
        if delta < 0:
            n = node
            while n is not self.root:
                if n.ref <= 0:
                    return ERR_STATE
                n = n.parent
        self._lock(node, delta)
        return OK

    def allocate(self, rows, cached, device) -> int:
        P = self.P
        up = lambda x: -(-x // P) * P
        total = 0
        for r, c, d in zip(rows, cached, device):
            if not self.row_used[r] or c < 0 or d < c or d > self.max_len:
                return ERR_ARG
            if self.row_len[r] > up(c):
                return ERR_STATE
            total += up(d) // P - up(c) // P
        if total > len(self.free_pages):
            self._evict(total - len(self.free_pages))
        if total > len(self.free_pages):
            return ERR_FULL
        for r, c, d in zip(rows, cached, device):
            for j in range(up(c), up(d), P):
                s = self.free_pages.popleft()
                self.table[r, j:j + P] = np.arange(s, s + P, dtype=np.int32)
            self.row_len[r] = max(self.row_len[r], up(d))
        return OK

    def cache_req(self, row: int, ids, cached_len: int, old: Node, finished: bool):
        """-> (status, new handle node, its length)"""
        if not self.row_used[row] or cached_len > self.row_len[row] or old.depth > cached_len:
            return ERR_ARG, None, 0
        t = self.table[row]
        n_al = cached_len - cached_len % self.P
        node, matched = self._walk(ids, n_al)
        if matched < n_al:
            leaf = self._new_node()
            leaf.parent = node
            leaf.key = [int(x) for x in ids[matched:n_al]]
            leaf.value = [int(x) for x in t[matched:n_al]]
            leaf.depth = n_al
            leaf.stamp = self.clock
            node.children[tuple(leaf.key[:self.P])] = leaf
            self.evictable += n_al - matched
            node = leaf
        self._lock(old, -1)
        if matched > old.depth:
            self._free_run(t, old.depth, matched)
            t[old.depth:matched] = self._path(node)[old.depth:matched]
        if finished:
            self._free_run(t, n_al, self.row_len[row])
            self.row_len[row] = 0
        else:
            self._lock(node, +1)
        return OK, node, n_al

    def release(self, row: int, node: Node) -> int:
        st = self.lock(node, -1)
        if st != OK:
            return st
        self._free_run(self.table[row], node.depth, self.row_len[row])
        self.row_len[row] = 0
        return OK

    def evict(self, pages: int) -> int:
        return self._evict(pages)

    def stats(self):
        n = 0
        stack = [self.root]
        while stack:
            nd = stack.pop()
            n += len(nd.children)
            stack.extend(nd.children.values())
        return [len(self.free_pages), self.evictable, self.protected, n, len(self.free_rows),
                self.clock]

    # -- inspection ---------------------------------------------------------
    def sequences(self) -> list[tuple[tuple, tuple]]:
        """(ids, slots) of every root-to-node path."""
        out, stack = [], [(self.root, (), ())]
        while stack:
            nd, ids, slots = stack.pop()
            for ch in nd.children.values():
                ci, cs = ids + tuple(ch.key), slots + tuple(ch.value)
                out.append((ci, cs))
                stack.append((ch, ci, cs))
        return out
