"""Paged-KV attention for MI355X (gfx950): store_kv, paged decode, extend, merge.

The compute lives in ``libmsgl.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/msgl.h``); this package is the thin ctypes binding.
"""

from .binding import (  # noqa: F401
    MsglError,
    PlannedCall,
    plan_store_kv,
    plan_paged_decode,
    plan_store_kv_paged_decode,
    plan_paged_extend,
    load,
    version,
    store_kv,
    paged_decode,
    store_kv_paged_decode,
    store_kv_paged_decode_noalloc,
    paged_decode_workspace_size,
    paged_extend,
    paged_extend_workspace_size,
    merge_states,
    embedding_gather,
    rope_cos_sin_cache,
    qk_norm_rope_store,
    plan_qk_norm_rope_store,
    plan_embedding_gather,
    alloc_workspace,
    DecodeGraph,
)
from ._build import LIB_PATH  # noqa: F401
from .kvcache import KVCache, compare_key  # noqa: F401
