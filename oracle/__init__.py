"""CPU oracle for paged-KV attention — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain reference that the HIP library is checked
against.  Only the test-suite, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import it.  The product path never calls
it and shares no code with it: the two meet only at the seeded input arrays
produced by the ``workloads`` package.

Everything here is written from the definitions on the source pages
(cited per function) and computes in float64 after an exact bf16 -> f64
upcast.  See ``oracle/attention.py``, ``oracle/embedding.py`` and
``oracle/prologue.py`` for the
functions and their pins (the ``tests/test_oracle_*.py`` files); every
function is pinned.  ``oracle/radix.py`` is the integer host logic of the
KV cache manager (page allocator + radix prefix cache), pinned in
``tests/test_oracle_radix.py``.
"""

from .radix import KVCacheOracle, compare_key  # noqa: F401

from .embedding import embedding_gather  # noqa: F401
from .prologue import rope_cache, rms_norm, rope, qk_norm_rope_store  # noqa: F401
from .attention import (  # noqa: F401
    bf16_to_f64,
    f64_to_bf16_rne,
    store_kv,
    gather_rows,
    attend_one,
    paged_decode,
    paged_decode_partial,
    paged_extend,
    merge_states,
    paged_decode_split,
    token_table_to_page_ids,
    page_ids_to_token_table,
    kv_bytes_per_token,
    kv_bytes_per_page,
    pool_pages_for_budget,
)
