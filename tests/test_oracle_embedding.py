"""Pins of the embedding-gather oracle (CPU).

The gather is a definition (row copy with a vocabulary-range mask), so the
pins are independent restatements of what that definition fixes:
* a hand-built table where row r holds the value r: the output is the id
  minus the shard start, or 0 outside the shard;
* numpy fancy indexing on an unsharded table;
* the tensor-parallel property the mask exists for [MSCA §4.7.8]: summing
  the masked gathers of every vocabulary shard gives the unsharded gather;
* bit-exactness for bf16 payloads (NaN / inf / signed-zero bit patterns are
  copied untouched).
"""

import numpy as np
import pytest

import oracle


def test_row_value_table_and_mask():
    table = np.repeat(np.arange(10, dtype=np.float32)[:, None], 3, axis=1)   # row r = [r, r, r]
    ids = np.array([0, 3, 9, 10, -1, 5, 12, 7])
    out = oracle.embedding_gather(table, ids, vocab_start=3)                   # rows = vocab 3..12
    want = np.array([0, 0, 6, 7, 0, 2, 9, 4], dtype=np.float32)
    assert np.array_equal(out, np.repeat(want[:, None], 3, axis=1))


def test_unsharded_equals_fancy_indexing():
    rng = np.random.default_rng(0)
    table = rng.integers(0, 1 << 16, size=(50, 33), dtype=np.uint16)
    ids = rng.integers(0, 50, size=200)
    assert np.array_equal(oracle.embedding_gather(table, ids), table[ids])


@pytest.mark.parametrize("shards", [1, 2, 3, 8])
def test_sum_over_vocab_shards_is_the_full_gather(shards):
    rng = np.random.default_rng(shards)
    V, H = 97, 16
    full = rng.standard_normal((V, H)).astype(np.float32)
    ids = rng.integers(0, V, size=300)
    bounds = np.linspace(0, V, shards + 1).astype(int)
    total = np.zeros((len(ids), H), np.float32)
    hits = np.zeros(len(ids), int)
    for a, b in zip(bounds[:-1], bounds[1:]):
        part = oracle.embedding_gather(full[a:b], ids, vocab_start=a)
        hits += np.any(part != 0, axis=1)
        total += part
    assert np.array_equal(total, full[ids])
    assert np.all(hits <= 1)          # exactly one shard contributes each row


def test_bf16_bits_copied_untouched():
    table = np.array([[0x7FC0, 0x7F80, 0x8000, 0x0001], [0xFF80, 0x0000, 0x3F80, 0xBF80]], np.uint16)
    out = oracle.embedding_gather(table, np.array([1, 0, 1]))
    assert np.array_equal(out, table[[1, 0, 1]])
    assert out.dtype == np.uint16


def test_empty_and_out_of_range():
    table = np.ones((4, 2), np.float32)
    assert oracle.embedding_gather(table, np.array([], dtype=np.int64)).shape == (0, 2)
    out = oracle.embedding_gather(table, np.array([4, -5, 2**40]))
    assert not out.any()


MUTANTS = [
    ("0 <= local < rows", "0 <= local <= rows"),            # off-by-one upper bound
    ("int(t) - int(vocab_start)", "int(t) + int(vocab_start)"),   # sign of the shard offset
    ("0 <= local < rows", "local < rows"),                   # no lower bound (negative wraps)
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_planted_mistakes_are_caught(old, new):
    import os
    import types
    src = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "embedding.py")).read()
    assert old in src
    mod = types.ModuleType("embedding_mutant")
    exec(compile(src.replace(old, new, 1), "embedding_mutant", "exec"), mod.__dict__)
    caught = False
    try:
        table = np.repeat(np.arange(10, dtype=np.float32)[:, None], 3, axis=1)
        ids = np.array([0, 3, 9, 10, -1, 5, 12, 7, 13])
        out = mod.embedding_gather(table, ids, vocab_start=3)
        want = np.array([0, 0, 6, 7, 0, 2, 9, 4, 0], dtype=np.float32)
        caught = not np.array_equal(out, np.repeat(want[:, None], 3, axis=1))
    except IndexError:
        caught = True
    assert caught
