"""Algorithmic work of one call: the bytes and FLOPs the method must spend.

These are the numerators of the roofline figures.  They count what the
definition needs, not what a kernel happens to do:

* decode reads every *distinct* K and V row its requests reference once
  (a slot shared by several requests counts once), walks one 4-byte page
  table entry per (request, page) — per token at page_size 1 — reads q and
  writes the output, and
  writes an fp32 log-sum-exp per (request, q head) when asked to;
* extend performs two multiply-adds per head dimension for each
  (query, key) pair the causal mask keeps, in each of QK^T and PV;
* store_kv reads and writes each new K and V row once.
"""

from __future__ import annotations

import numpy as np


def unique_kv_slots(page_table, req_rows, lens) -> int:
    parts = [np.asarray(page_table[int(req_rows[r]), : int(L)]) for r, L in enumerate(lens)]
    if not parts:
        return 0
    return int(np.unique(np.concatenate(parts)).size)


def decode_bytes(page_table, req_rows, seq_lens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, dtype_bytes: int = 2, with_lse: bool = True,
                 page_size: int = 1) -> int:
    B = len(seq_lens)
    kv = unique_kv_slots(page_table, req_rows, seq_lens) * 2 * num_kv_heads * head_dim * dtype_bytes
    lens = np.asarray(seq_lens, dtype=np.int64)
    walked = 4 * int(np.sum((lens + page_size - 1) // page_size))
    qo = 2 * B * num_q_heads * head_dim * dtype_bytes
    return kv + walked + qo + (4 * B * num_q_heads if with_lse else 0)


def decode_kv_bytes(page_table, req_rows, seq_lens, num_kv_heads: int, head_dim: int,
                    dtype_bytes: int = 2) -> int:
    """Distinct K+V bytes only (the headline numerator)."""
    return unique_kv_slots(page_table, req_rows, seq_lens) * 2 * num_kv_heads * head_dim * dtype_bytes


def causal_pairs(prefix_lens, extend_lens) -> int:
    """sum_r  E_r * P_r + E_r (E_r + 1) / 2  (query i sees P + i + 1 keys)."""
    total = 0
    for P, E in zip(prefix_lens, extend_lens):
        P, E = int(P), int(E)
        total += E * P + E * (E + 1) // 2
    return total


def extend_flops(prefix_lens, extend_lens, num_q_heads: int, head_dim: int) -> int:
    return 4 * num_q_heads * head_dim * causal_pairs(prefix_lens, extend_lens)


def store_bytes(n_rows: int, num_kv_heads: int, head_dim: int, dtype_bytes: int = 2,
                index_bytes: int = 8) -> int:
    row = num_kv_heads * head_dim * dtype_bytes
    return n_rows * (4 * row + index_bytes)
