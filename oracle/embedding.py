"""Plain CPU oracle for the vocabulary-sharded embedding gather.

TEST INFRASTRUCTURE ONLY — see ``oracle/__init__.py``.  Nothing in the
library imports this module; it imports nothing from the library.

Source: "Mini-SGLang complete analysis" (blog.rzhang-lab.cn):
  - §4.9.3, the call chain of one ``indexing(weights, ids, vocab_range)``
    call: the embedding gather copies one table row per token id;
  - §4.7.8, the sharding map: ``embed_tokens`` is split along the vocabulary
    dimension across tensor-parallel ranks and combined by masked indexing
    followed by an all-reduce.

Reading: a rank holding vocabulary rows
``[vocab_start, vocab_start + rows)`` writes, for token id ``t``, row
``t - vocab_start`` of its table when ``t`` falls in that range and a row of
zeros otherwise, so that the sum over ranks (the all-reduce) is the full
table's row.  Rows are copied bit for bit (no arithmetic).
"""

from __future__ import annotations

import numpy as np


def embedding_gather(weights: np.ndarray, ids: np.ndarray, vocab_start: int = 0) -> np.ndarray:
    """out[i] = weights[ids[i] - vocab_start] if that row exists, else zeros.

    ``weights``: [rows, hidden] array of any element type (bf16 bits as
    uint16, or float32); ``ids``: [n] integer token ids.  Returns a new
    [n, hidden] array of the same element type.  [MSCA §4.9.3, §4.7.8]
    """
    rows = weights.shape[0]
    out = np.zeros((len(ids),) + weights.shape[1:], dtype=weights.dtype)
    for i, t in enumerate(np.asarray(ids, dtype=np.int64)):
        local = int(t) - int(vocab_start)
        if 0 <= local < rows:
            out[i] = weights[local]
    return out
