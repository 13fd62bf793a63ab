"""Seeded request trace for the host KV cache manager (inputs only).

A serving-like mix in the shape the pages describe for prefix reuse: many
requests open with one of a few shared system prompts (the "100 requests with
the same 4096-token system prompt" scenario of "Mini-SGLang complete
analysis" §1.4), followed by a request-specific part, then a number of decode
steps.  Prompt popularity is Zipf-like.  Token ids are int32.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class KVTrace:
    prompts: list          # list of int32 arrays (system prompt + own part)
    decode_steps: np.ndarray
    page_size: int
    num_slots: int
    max_rows: int
    max_len: int


def kv_trace(seed: int = 7, num_requests: int = 1024, num_system: int = 32,
             system_len: int = 1024, user_len: int = 256, decode_len: int = 64,
             page_size: int = 16, num_slots: int = 262144, max_rows: int = 128,
             vocab: int = 32000, zipf_s: float = 1.1) -> KVTrace:
    rng = np.random.Generator(np.random.PCG64(seed))
    systems = [rng.integers(0, vocab, system_len, dtype=np.int64).astype(np.int32)
               for _ in range(num_system)]
    w = 1.0 / np.arange(1, num_system + 1) ** zipf_s
    pick = rng.choice(num_system, size=num_requests, p=w / w.sum())
    prompts = []
    for k in range(num_requests):
        own = rng.integers(0, vocab, int(rng.integers(user_len // 2, user_len + 1)), dtype=np.int64)
        prompts.append(np.concatenate([systems[pick[k]], own.astype(np.int32)]))
    steps = rng.integers(decode_len // 2, decode_len + 1, num_requests)
    max_len = -(-(system_len + user_len + decode_len) // page_size) * page_size
    return KVTrace(prompts, steps, page_size, num_slots, max_rows, max_len)


def drive(kv, trace: KVTrace, token_rng_seed: int = 0):
    """Run a trace through a manager with the binding's / oracle's method
    names: continuous batching with prefix matching at admission, the whole
    prompt cached after prefill, one batched one-token allocation per decode
    step, and caching on finish.  Returns counts of what happened."""
    rng = np.random.Generator(np.random.PCG64(token_rng_seed))
    pending = list(range(len(trace.prompts)))
    running = {}                     # row -> [req, ids list, len, handle, steps left]
    stats = {"admitted": 0, "matched_tokens": 0, "prompt_tokens": 0, "decode_tokens": 0,
             "deferred": 0, "calls": 0}
    while pending or running:
        # admission
        while pending and len(running) < trace.max_rows:
            k = pending[0]
            ids = trace.prompts[k]
            st, row = kv.alloc_row()
            stats["calls"] += 1
            if st != 0:
                break
            st, cl, h = kv.match(ids, row)
            kv.lock(h, 1)
            st = kv.allocate([row], [cl], [len(ids)])
            stats["calls"] += 3
            if st != 0:
                kv.release(row, h)
                kv.free_row(row)
                stats["calls"] += 2
                stats["deferred"] += 1
                break
            st, h2, _ = kv.cache_req(row, ids, len(ids), h, False)
            stats["calls"] += 1
            pending.pop(0)
            running[row] = [k, list(ids), len(ids), h2, int(trace.decode_steps[k])]
            stats["admitted"] += 1
            stats["matched_tokens"] += cl
            stats["prompt_tokens"] += len(ids)
        # one decode step for everyone
        rows = list(running)
        if rows:
            c = [running[r][2] for r in rows]
            st = kv.allocate(rows, c, [x + 1 for x in c])
            stats["calls"] += 1
            if st == 0:
                for r in rows:
                    q = running[r]
                    q[1].append(int(rng.integers(0, 32000)))
                    q[2] += 1
                    q[4] -= 1
                stats["decode_tokens"] += len(rows)
            else:
                # out of pages: the newest request gives its pages back and waits
                r = rows[-1]
                q = running.pop(r)
                kv.release(r, q[3])
                kv.free_row(r)
                pending.insert(0, q[0])
                stats["calls"] += 2
        for r in [r for r in rows if r in running and running[r][4] <= 0]:
            q = running.pop(r)
            kv.cache_req(r, q[1], q[2], q[3], True)
            kv.free_row(r)
            stats["calls"] += 2
    return stats
