"""Seeded synthetic inputs for paged-KV attention.

This module only *draws* inputs: lengths, a slot (or page) permutation, the
pool contents, queries and the new K/V rows.  It holds none of the attention
arithmetic, imports nothing from the library or the oracle, and is the one
piece of code that both sides (GPU tests/bench and the CPU oracle) share.

Recipe (fixed, so every run of every config sees the same bits):

* ``rng = numpy.random.Generator(PCG64(seed))`` draws, in this order:
  lengths, the slot (page) permutation, q, k_new, v_new, then the
  request-to-table-row permutation.
* The K pool and V pool are drawn in chunks of ``CHUNK_VALUES`` values; chunk
  ``c`` of stream ``s`` (1 = K, 2 = V) uses
  ``PCG64(SeedSequence([seed, s, c]))``, so the result does not depend on the
  number of worker threads.
* Every value is standard normal float32 rounded to bf16 (nearest, ties to
  even) and kept as raw ``uint16`` bits.
* Each request's own tokens take the next consecutive segment of the
  permutation; a shared prefix takes the first segment and is reused
  verbatim by every request that shares it.  With page_size P the
  permutation is over pages and token ``j`` of a request sits in slot
  ``page[j // P] * P + j % P``; every request's own part starts on a page
  boundary.
* The page table has one row per request plus one spare row; requests are
  mapped to rows by a random permutation, and unused entries point at a
  valid slot so that a stray read returns wrong values instead of faulting.
* Pool size, unless a config fixes it: ``round_up(1.25 * unique tokens,
  65536)`` slots.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK_VALUES = 1 << 22
STREAM_K = 1
STREAM_V = 2


# ---------------------------------------------------------------------------
# value generation
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even), as bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def random_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard-normal bf16 bits drawn from ``rng``."""
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16_stream(seed: int, stream: int, count: int) -> np.ndarray:
    """``count`` bf16 bits from the chunked parallel stream ``(seed, stream)``."""
    out = np.empty(count, dtype=np.uint16)
    nchunks = -(-count // CHUNK_VALUES)

    def fill(c: int) -> None:
        lo = c * CHUNK_VALUES
        hi = min(count, lo + CHUNK_VALUES)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        out[lo:hi] = f32_to_bf16_bits(g.standard_normal(hi - lo, dtype=np.float32))

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def round_up(x: int, m: int) -> int:
    return -(-x // m) * m


# ---------------------------------------------------------------------------
# the input bundle
# ---------------------------------------------------------------------------

@dataclass
class PagedInputs:
    """One synthetic batch: pool, table, store rows, decode and extend parts.

    All bf16 tensors are raw ``uint16`` bits.  ``k_pool``/``v_pool`` hold the
    pool *before* the new rows are stored.
    """
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    sm_scale: float
    k_pool: np.ndarray                 # [num_slots, Hkv, D] uint16
    v_pool: np.ndarray
    page_table: np.ndarray             # [rows, W] int32, token granular
    out_loc: np.ndarray                # [n] int64
    k_new: np.ndarray                  # [n, Hkv, D] uint16
    v_new: np.ndarray
    dec_req_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    dec_seq_lens: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    dec_q: np.ndarray | None = None    # [Bd, Hq, D] uint16
    ext_req_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    ext_prefix_lens: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    ext_extend_lens: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    ext_q_offsets: np.ndarray = field(default_factory=lambda: np.zeros(1, np.int32))
    ext_q: np.ndarray | None = None    # [T, Hq, D] uint16
    notes: dict = field(default_factory=dict)

    @property
    def num_slots(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def num_decode(self) -> int:
        return int(len(self.dec_seq_lens))

    @property
    def num_extend(self) -> int:
        return int(len(self.ext_extend_lens))

    @property
    def ext_tokens(self) -> int:
        return int(self.ext_q_offsets[-1]) if len(self.ext_q_offsets) else 0


# ---------------------------------------------------------------------------
# generic builder
# ---------------------------------------------------------------------------

def build_inputs(name: str, *, seed: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, page_size: int, decode_lens, extend_specs,
                 shared_prefix: int = 0, shared_by=(), num_slots: int | None = None,
                 sm_scale: float | None = None, lengths_rng=None,
                 table_pad: int = 17) -> PagedInputs:
    """Draw a batch of decode and extend requests over one paged pool.

    ``decode_lens``: kv length of each decode request (including its new
    token).  ``extend_specs``: ``(prefix_len, extend_len)`` per extend request.
    Extend requests come first in table order, then decode requests.
    ``shared_by``: request indices (in that order) whose first
    ``shared_prefix`` tokens are one common segment.  ``lengths_rng``: the
    generator already used to draw the lengths (``None`` -> a fresh one).
    """
    rng = lengths_rng if lengths_rng is not None else np.random.Generator(np.random.PCG64(seed))
    P = page_size
    ext = [(int(p), int(e)) for p, e in extend_specs]
    dec = [int(x) for x in decode_lens]
    kv_lens = [p + e for p, e in ext] + dec
    B = len(kv_lens)
    shared = set(int(i) for i in shared_by)
    if shared_prefix % P:
        raise ValueError("a shared prefix must be page aligned")
    for i in shared:
        if kv_lens[i] < shared_prefix:
            raise ValueError("request shorter than the shared prefix")
    own = [L - (shared_prefix if i in shared else 0) for i, L in enumerate(kv_lens)]
    pages_needed = (shared_prefix // P if shared else 0) + sum(-(-o // P) for o in own)
    unique_tokens = pages_needed * P
    if num_slots is None:
        num_slots = round_up(int(math.ceil(1.25 * unique_tokens)), 65536)
    num_pages = num_slots // P
    if num_pages < pages_needed:
        raise ValueError("pool too small")

    perm = rng.permutation(num_pages).astype(np.int64)
    cursor = 0
    shared_pages = np.zeros(0, np.int64)
    if shared:
        shared_pages = perm[: shared_prefix // P]
        cursor = shared_prefix // P
    W = max(kv_lens) + table_pad if kv_lens else 1
    rows = B + 1
    spare = int(perm[-1]) * P
    table = np.full((rows, W), spare, dtype=np.int64)
    req_tokens = []
    for i, L in enumerate(kv_lens):
        start = shared_prefix if i in shared else 0
        npg = -(-(L - start) // P)
        pages = perm[cursor: cursor + npg]
        cursor += npg
        page_list = np.concatenate([shared_pages, pages]) if i in shared else pages
        j = np.arange(L, dtype=np.int64)
        req_tokens.append(page_list[j // P] * P + j % P)

    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    k_pool = normal_bf16_stream(seed, STREAM_K, num_slots * Hkv * D).reshape(num_slots, Hkv, D)
    v_pool = normal_bf16_stream(seed, STREAM_V, num_slots * Hkv * D).reshape(num_slots, Hkv, D)

    n_ext_tok = sum(e for _, e in ext)
    ext_q = random_bf16(rng, (n_ext_tok, Hq, D)) if ext else None
    dec_q = random_bf16(rng, (len(dec), Hq, D)) if dec else None
    n_new = n_ext_tok + len(dec)
    k_new = random_bf16(rng, (n_new, Hkv, D))
    v_new = random_bf16(rng, (n_new, Hkv, D))
    row_of = rng.permutation(B).astype(np.int32)

    for i in range(B):
        table[row_of[i], : kv_lens[i]] = req_tokens[i]

    out_loc = []
    for i, (p, e) in enumerate(ext):
        out_loc.extend(req_tokens[i][p: p + e].tolist())
    for k, L in enumerate(dec):
        out_loc.append(int(req_tokens[len(ext) + k][L - 1]))

    q_off = np.zeros(len(ext) + 1, np.int32)
    q_off[1:] = np.cumsum([e for _, e in ext]) if ext else []
    inp = PagedInputs(
        name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
        sm_scale=float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(D)),
        k_pool=k_pool, v_pool=v_pool, page_table=table.astype(np.int32),
        out_loc=np.asarray(out_loc, dtype=np.int64), k_new=k_new, v_new=v_new,
        dec_req_rows=row_of[len(ext):].copy(),
        dec_seq_lens=np.asarray(dec, np.int32),
        dec_q=dec_q,
        ext_req_rows=row_of[: len(ext)].copy(),
        ext_prefix_lens=np.asarray([p for p, _ in ext], np.int32),
        ext_extend_lens=np.asarray([e for _, e in ext], np.int32),
        ext_q_offsets=q_off,
        ext_q=ext_q,
    )
    uniq = int(np.unique(np.concatenate(req_tokens)).size) if req_tokens else 0
    inp.notes.update(unique_tokens=uniq, shared_prefix=shared_prefix,
                     shared_by=sorted(shared))
    return inp


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------

def config_c1(seed: int = 1) -> PagedInputs:
    """Tiny decode: Hq 16 / Hkv 8, lens 17/64/100/255, 1,024 slots."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return build_inputs("C1", seed=seed, num_q_heads=16, num_kv_heads=8,
                        head_dim=128, page_size=1, decode_lens=[17, 64, 100, 255],
                        extend_specs=[], num_slots=1024, lengths_rng=rng)


def config_c2(seed: int = 2) -> PagedInputs:
    """8B-class decode: Hq 32 / Hkv 8, B 64, lens U[512, 4096], 512K slots."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(512, 4097, 64)
    return build_inputs("C2", seed=seed, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, page_size=1, decode_lens=lens,
                        extend_specs=[], num_slots=524288, lengths_rng=rng)


C3_PREFIXES = (2048, 2048, 2048, 2048, 0, 1024, 4096, 8192)


def config_c3(seed: int = 3) -> PagedInputs:
    """Chunked-prefill extend: 8 requests, 4 share one 2,048-slot prefix."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ext_lens = rng.integers(512, 2049, 8)
    specs = list(zip(C3_PREFIXES, ext_lens))
    return build_inputs("C3", seed=seed, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, page_size=1, decode_lens=[],
                        extend_specs=specs, shared_prefix=2048,
                        shared_by=(0, 1, 2, 3), lengths_rng=rng)


def c4_lengths(rng: np.random.Generator, batch: int = 256) -> np.ndarray:
    raw = rng.lognormal(math.log(2048.0), 1.0, batch)
    return np.clip(np.rint(raw), 1024, 32768).astype(np.int64)


def config_c4(seed: int = 4) -> PagedInputs:
    """Long-tail decode: Hq 64 / Hkv 8, B 256, lognormal lens in [1K, 32K]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = c4_lengths(rng)
    return build_inputs("C4", seed=seed, num_q_heads=64, num_kv_heads=8,
                        head_dim=128, page_size=1, decode_lens=lens,
                        extend_specs=[], lengths_rng=rng)


def config_c5(seed: int = 5, page_size: int = 1) -> PagedInputs:
    """Mixed batch: one extend (6,144 + 2,048) and 127 decode requests.

    64 of the 128 requests share one 1,024-token prefix: the extend request
    and the first 63 decode requests (in order) whose length is >= 1,025.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = rng.integers(256, 8193, 127)
    sharers = [0]
    for k, L in enumerate(lens):
        if len(sharers) == 64:
            break
        if L >= 1025:
            sharers.append(1 + k)
    return build_inputs(f"C5{'a' if page_size == 1 else 'b'}", seed=seed,
                        num_q_heads=32, num_kv_heads=8, head_dim=128,
                        page_size=page_size, decode_lens=lens,
                        extend_specs=[(6144, 2048)], shared_prefix=1024,
                        shared_by=sharers, lengths_rng=rng)


CONFIGS = {
    "C1": config_c1,
    "C2": config_c2,
    "C3": config_c3,
    "C4": config_c4,
    "C5a": lambda: config_c5(page_size=1),
    "C5b": lambda: config_c5(page_size=16),
}


def make_config(name: str) -> PagedInputs:
    return CONFIGS[name]()


# ---------------------------------------------------------------------------
# small shapes for tests
# ---------------------------------------------------------------------------

def small_decode(seed: int, num_q_heads: int, num_kv_heads: int, seq_lens,
                 page_size: int = 1, num_slots: int | None = None,
                 shared_prefix: int = 0, shared_by=(), head_dim: int = 128,
                 sm_scale: float | None = None) -> PagedInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    return build_inputs(f"decode-{seed}", seed=seed, num_q_heads=num_q_heads,
                        num_kv_heads=num_kv_heads, head_dim=head_dim,
                        page_size=page_size, decode_lens=seq_lens,
                        extend_specs=[], num_slots=num_slots,
                        shared_prefix=shared_prefix, shared_by=shared_by,
                        sm_scale=sm_scale, lengths_rng=rng)


def small_extend(seed: int, num_q_heads: int, num_kv_heads: int, specs,
                 page_size: int = 1, num_slots: int | None = None,
                 decode_lens=(), shared_prefix: int = 0, shared_by=(),
                 head_dim: int = 128, sm_scale: float | None = None) -> PagedInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    return build_inputs(f"extend-{seed}", seed=seed, num_q_heads=num_q_heads,
                        num_kv_heads=num_kv_heads, head_dim=head_dim,
                        page_size=page_size, decode_lens=decode_lens,
                        extend_specs=specs, num_slots=num_slots,
                        shared_prefix=shared_prefix, shared_by=shared_by,
                        sm_scale=sm_scale, lengths_rng=rng)
