"""Plain float64 CPU oracle for attention over a paged KV pool.

TEST INFRASTRUCTURE ONLY — see ``oracle/__init__.py``.  Nothing in the
library imports this module; it imports nothing from the library.

Sources (five web pages about the mini-sglang inference engine):

* "Mini-SGLang complete analysis" (blog.rzhang-lab.cn), cited as [MSCA §x]:
  - §1.3  KV cache size per token (the 128 KB worked figure);
  - §1.4  paged KV cache: one pool of fixed-size pages plus a per-request
          page table that the attention kernel reads through;
  - §4.2.3 the request length fields (cached_len, device_len, extend_len);
  - §4.4.3 the pool is one tensor (K/V, layer, page, slot-in-page, kv head,
          head dim), flattened per layer to (pages*page_size, kv heads, dim)
          and written by ``store_kv`` at ``out_loc``;
  - §4.5.3 grouped-query attention: ratio = q heads // kv heads;
  - §4.6.4 the global page table is always kept at page_size = 1
          (token granularity); page-granular backends take every
          page_size-th column and divide by page_size;
  - §4.6.7 the attention layer stores the new K/V first, then runs the
          paged kernel;
  - §4.9.4 the store kernel's contract: pools [-1, D], new rows [L, D],
          indices [L] int32 or int64;
  - §5.2  the worked KV-budget arithmetic (442k slots, 6,912 pages).
* "Deep dive into mini-sglang: chunked prefill and overlap scheduling"
  (yunpan.plus), cited as [DDMS], section on chunked prefill: every chunk of
  a long prompt reuses the KV of the chunks before it.

Readings where the pages are silent:

* scores are ``sm_scale * (q . k)`` with the natural exponential; no
  soft-cap, no ALiBi, no window;
* extend is causal and bottom-right aligned: query ``i`` of a request with
  prefix ``P`` sees keys ``0 .. P+i``;
* a decode ``seq_len`` already counts the token just stored;
* q head ``h`` uses kv head ``h // ratio`` (contiguous groups);
* the log-sum-exp is in natural-log units;
* an empty key range gives output 0 and lse = -inf;
* the split-KV merge of partial states (o_s, lse_s) is
  ``o = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M)``,
  ``lse = M + ln sum_s exp(lse_s - M)`` with ``M = max_s lse_s`` — the pages
  do not describe split-KV at all; this is the identity that makes a split
  softmax equal the unsplit one.

All floating point is float64.  Inputs arrive as raw bf16 bit patterns
(``uint16`` arrays) and are upcast exactly.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_to_f64",
    "f64_to_bf16_rne",
    "store_kv",
    "gather_rows",
    "attend_one",
    "paged_decode",
    "paged_decode_partial",
    "paged_extend",
    "merge_states",
    "paged_decode_split",
    "token_table_to_page_ids",
    "page_ids_to_token_table",
    "kv_bytes_per_token",
    "kv_bytes_per_page",
    "pool_pages_for_budget",
]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> float64: a bf16 value is the top half of an IEEE fp32."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        bits = bits.view(np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit pattern, round to nearest, ties to even.

    One rounding step straight from float64 (no detour through float32,
    which could round twice).  bf16 keeps 8 significant bits and fp32's
    exponent range; values below 2**-126 round on the subnormal grid 2**-133.
    NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    for i, v in enumerate(flat):
        if math.isnan(v):
            res[i] = 0x7FC0
            continue
        if v == 0.0 or math.isinf(v):
            res[i] = np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16
            continue
        e = math.floor(math.log2(abs(v)))
        # guard log2 rounding at exact powers of two
        if 2.0 ** e > abs(v):
            e -= 1
        elif 2.0 ** (e + 1) <= abs(v):
            e += 1
        e = max(e, -126)
        q = 2.0 ** (e - 7)             # spacing of bf16 values near v
        r = round(v / q) * q           # Python round(): ties to even
        if abs(r) >= 2.0 ** 128:
            r = math.copysign(math.inf, v)
        res[i] = np.array([r], dtype=np.float32).view(np.uint32)[0] >> 16
    return out


# ---------------------------------------------------------------------------
# a1: store_kv  [MSCA §4.4.3, §4.6.7, §4.9.4]
# ---------------------------------------------------------------------------

def store_kv(k_pool: np.ndarray, v_pool: np.ndarray,
             k_new: np.ndarray, v_new: np.ndarray,
             out_loc: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Row scatter of new K/V into the flattened per-layer pool.

    ``k_pool``/``v_pool`` are raw bf16 bits ``[num_slots, Hkv, D]`` (the
    per-layer view of [MSCA §4.4.3]); ``k_new``/``v_new`` are ``[n, Hkv, D]``;
    ``out_loc`` holds ``n`` distinct slot indices.  Row ``i`` of the new
    tensors lands in slot ``out_loc[i]``; every other slot keeps its bytes.
    Returns new arrays (the inputs are not modified).
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for i in range(len(out_loc)):
        slot = int(out_loc[i])
        k_out[slot] = k_new[i]
        v_out[slot] = v_new[i]
    return k_out, v_out


# ---------------------------------------------------------------------------
# a2/a3: the page-table walk and the row gather  [MSCA §1.4, §4.6.4]
# ---------------------------------------------------------------------------

def gather_rows(pool: np.ndarray, page_table_row: np.ndarray,
                begin: int, end: int, kv_head: int) -> np.ndarray:
    """Materialise keys ``begin .. end-1`` of one request for one kv head.

    Token ``j`` of the request lives in slot ``page_table_row[j]``
    (token-granular table, [MSCA §4.6.4]).  Returns float64 ``[end-begin, D]``
    in logical token order.
    """
    slots = [int(page_table_row[j]) for j in range(begin, end)]
    if not slots:
        return np.zeros((0, pool.shape[-1]), dtype=np.float64)
    return bf16_to_f64(pool[slots, kv_head, :])


# ---------------------------------------------------------------------------
# a4: softmax attention of one query vector
# ---------------------------------------------------------------------------

def attend_one(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
               sm_scale: float) -> tuple[np.ndarray, float]:
    """softmax(sm_scale * keys @ q) @ values, and its log-sum-exp.

    ``q`` [D], ``keys``/``values`` [L, D] float64.  With L = 0 the result is
    the zero vector and lse = -inf (an empty softmax has no mass).
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64), -math.inf
    s = sm_scale * (keys @ q)
    m = float(np.max(s))
    p = np.exp(s - m)
    denom = float(np.sum(p))
    out = (p @ values) / denom
    lse = m + math.log(denom)
    return out, lse


# ---------------------------------------------------------------------------
# a4: paged GQA decode  [MSCA §1.2, §1.4, §4.5.3, §4.6.7]
# ---------------------------------------------------------------------------

def paged_decode_partial(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                         page_table: np.ndarray, req_rows, seq_lens,
                         sm_scale: float, num_kv_heads: int,
                         begins, ends) -> tuple[np.ndarray, np.ndarray]:
    """Decode attention of each request over its keys ``begins[r] .. ends[r]-1``.

    ``q`` bf16 bits ``[B, Hq, D]``; pools bf16 bits ``[num_slots, Hkv, D]``;
    ``page_table`` int ``[rows, W]``; request ``r`` uses table row
    ``req_rows[r]`` (identity when ``None``).  ``seq_lens`` is accepted for
    symmetry and bounds ``ends``.  Returns float64 ``out [B, Hq, D]`` and
    ``lse [B, Hq]``.
    """
    B, Hq, D = q.shape
    ratio = Hq // num_kv_heads
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -math.inf, dtype=np.float64)
    qf = bf16_to_f64(q)
    for r in range(B):
        row = r if req_rows is None else int(req_rows[r])
        b, e = int(begins[r]), int(ends[r])
        assert 0 <= b <= e <= int(seq_lens[r])
        for g in range(num_kv_heads):
            keys = gather_rows(k_pool, page_table[row], b, e, g)
            vals = gather_rows(v_pool, page_table[row], b, e, g)
            for h in range(g * ratio, (g + 1) * ratio):
                out[r, h], lse[r, h] = attend_one(qf[r, h], keys, vals, sm_scale)
    return out, lse


def paged_decode(q, k_pool, v_pool, page_table, req_rows, seq_lens,
                 sm_scale: float, num_kv_heads: int):
    """One query token per request over all ``seq_lens[r]`` cached keys.

    The new token's K/V were stored before the call ([MSCA §4.6.7]), so
    ``seq_lens[r]`` includes it.  Returns float64 ``(out [B,Hq,D], lse [B,Hq])``.
    """
    B = q.shape[0]
    return paged_decode_partial(q, k_pool, v_pool, page_table, req_rows,
                                seq_lens, sm_scale, num_kv_heads,
                                [0] * B, [int(x) for x in seq_lens])


# ---------------------------------------------------------------------------
# a5: merge of partial attention states  (pages silent; see module doc)
# ---------------------------------------------------------------------------

def merge_states(part_out: np.ndarray, part_lse: np.ndarray):
    """Combine S partial results over disjoint key sets.

    ``part_out`` [S, ..., D] float, ``part_lse`` [S, ...] float (natural log).
    Each part is a normalised softmax output over its own keys with its own
    log-sum-exp.  Parts with lse = -inf carry no mass.  If every part is
    empty the result is 0 with lse = -inf.
    """
    part_out = np.asarray(part_out, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    S = part_lse.shape[0]
    rest = part_lse.shape[1:]
    out = np.zeros(part_out.shape[1:], dtype=np.float64)
    lse = np.full(rest, -math.inf, dtype=np.float64)
    for idx in np.ndindex(*rest) if rest else [()]:
        lses = [float(part_lse[(s,) + idx]) for s in range(S)]
        M = max(lses)
        if M == -math.inf:
            continue
        w = [math.exp(x - M) for x in lses]
        total = sum(w)
        acc = np.zeros(part_out.shape[-1], dtype=np.float64)
        for s in range(S):
            acc += w[s] * part_out[(s,) + idx]
        out[idx] = acc / total
        lse[idx] = M + math.log(total)
    return out, lse


def paged_decode_split(q, k_pool, v_pool, page_table, req_rows, seq_lens,
                       sm_scale: float, num_kv_heads: int, split_tokens: int):
    """Split-KV decode: contiguous key chunks of ``split_tokens``, then merge.

    Chunk ``c`` of request ``r`` covers keys ``[c*S, min((c+1)*S, L))``.
    Returns ``(out, lse, part_out, part_lse)``; parts past a request's end are
    empty (lse = -inf).
    """
    B, Hq, D = q.shape
    L = [int(x) for x in seq_lens]
    nparts = max(1, max((-(-x // split_tokens) for x in L), default=1))
    part_out = np.zeros((nparts, B, Hq, D), dtype=np.float64)
    part_lse = np.full((nparts, B, Hq), -math.inf, dtype=np.float64)
    for c in range(nparts):
        b = [min(c * split_tokens, x) for x in L]
        e = [min((c + 1) * split_tokens, x) for x in L]
        part_out[c], part_lse[c] = paged_decode_partial(
            q, k_pool, v_pool, page_table, req_rows, seq_lens, sm_scale,
            num_kv_heads, b, e)
    out, lse = merge_states(part_out, part_lse)
    return out, lse, part_out, part_lse


# ---------------------------------------------------------------------------
# a6: causal chunked-prefill extend  [DDMS chunked prefill; MSCA §4.2.3]
# ---------------------------------------------------------------------------

def paged_extend(q, k_pool, v_pool, page_table, req_rows, prefix_lens,
                 extend_lens, q_offsets, sm_scale: float, num_kv_heads: int,
                 query_subset=None, block_rows: int = 512):
    """Causal extend attention over a cached prefix plus the chunk itself.

    Request ``r`` has ``P = prefix_lens[r]`` keys already cached and
    ``E = extend_lens[r]`` new tokens whose K/V were stored first; its keys
    are ``page_table[row, 0 : P+E]``.  Query ``i`` (global row
    ``q_offsets[r] + i`` of ``q [T, Hq, D]``) sees keys ``0 .. P+i``.

    ``query_subset``: optional iterable of global query rows; only those rows
    are computed (the rest stay 0 / -inf).  Queries are processed in blocks
    of ``block_rows`` rows to bound memory.
    Returns float64 ``(out [T,Hq,D], lse [T,Hq])``.
    """
    T, Hq, D = q.shape
    ratio = Hq // num_kv_heads
    out = np.zeros((T, Hq, D), dtype=np.float64)
    lse = np.full((T, Hq), -math.inf, dtype=np.float64)
    wanted = None if query_subset is None else set(int(x) for x in query_subset)
    qf = bf16_to_f64(q)
    B = len(extend_lens)
    for r in range(B):
        row = r if req_rows is None else int(req_rows[r])
        P, E, base = int(prefix_lens[r]), int(extend_lens[r]), int(q_offsets[r])
        rows_i = [i for i in range(E) if wanted is None or base + i in wanted]
        if not rows_i:
            continue
        for g in range(num_kv_heads):
            keys = gather_rows(k_pool, page_table[row], 0, P + E, g)
            vals = gather_rows(v_pool, page_table[row], 0, P + E, g)
            for blk in range(0, len(rows_i), block_rows):
                ii = np.array(rows_i[blk:blk + block_rows])
                visible = P + ii + 1                       # keys 0..P+i
                for h in range(g * ratio, (g + 1) * ratio):
                    s = sm_scale * (qf[base + ii, h, :] @ keys.T)   # [n, P+E]
                    mask = np.arange(P + E)[None, :] < visible[:, None]
                    s = np.where(mask, s, -np.inf)
                    m = np.max(s, axis=1, keepdims=True)
                    p = np.where(mask, np.exp(s - m), 0.0)
                    denom = np.sum(p, axis=1, keepdims=True)
                    out[base + ii, h, :] = (p @ vals) / denom
                    lse[base + ii, h] = m[:, 0] + np.log(denom[:, 0])
    return out, lse


# ---------------------------------------------------------------------------
# page-size view of the token table  [MSCA §4.6.4]
# ---------------------------------------------------------------------------

def token_table_to_page_ids(row: np.ndarray, length: int, page_size: int) -> np.ndarray:
    """Page ids of one request: every page_size-th column, divided by page_size."""
    cols = list(range(0, length, page_size))
    return np.array([int(row[c]) // page_size for c in cols], dtype=np.int64)


def page_ids_to_token_table(page_ids, length: int, page_size: int) -> np.ndarray:
    """Inverse view: token ``j`` sits in slot ``page_ids[j // P] * P + j % P``."""
    return np.array([int(page_ids[j // page_size]) * page_size + j % page_size
                     for j in range(length)], dtype=np.int64)


# ---------------------------------------------------------------------------
# pool byte arithmetic  [MSCA §1.3, §4.4.3, §5.2]
# ---------------------------------------------------------------------------

def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int,
                       dtype_bytes: int) -> int:
    """K and V, every layer, every kv head, every dim of one token."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def kv_bytes_per_page(num_layers: int, page_size: int, num_kv_heads: int,
                      head_dim: int, dtype_bytes: int) -> int:
    """One page of the pool tensor across both K/V planes and all layers."""
    return page_size * kv_bytes_per_token(num_layers, num_kv_heads, head_dim,
                                          dtype_bytes)


def pool_pages_for_budget(budget_bytes: int, bytes_per_page: int) -> int:
    """Whole pages that fit a byte budget."""
    return budget_bytes // bytes_per_page
