"""The seeded input generators and the algorithmic byte/FLOP counts (CPU only)."""

import math

import numpy as np
import pytest

import workloads as W
from workloads import metrics


def test_chunked_stream_is_deterministic_and_thread_independent(monkeypatch):
    a = W.normal_bf16_stream(9, 1, 3 * W.synth.CHUNK_VALUES + 5)
    monkeypatch.setattr(W.synth, "_workers", lambda: 1)
    b = W.normal_bf16_stream(9, 1, 3 * W.synth.CHUNK_VALUES + 5)
    assert np.array_equal(a, b)
    c = W.normal_bf16_stream(9, 2, 1000)
    assert not np.array_equal(a[:1000], c)


def test_bf16_inputs_are_roughly_standard_normal():
    x = W.normal_bf16_stream(1, 1, 1 << 20)
    f = (x.astype(np.uint32) << 16).view(np.float32)
    assert abs(float(f.mean())) < 0.01 and abs(float(f.std()) - 1.0) < 0.01


def test_c1_structure():
    c = W.config_c1()
    assert c.num_slots == 1024 and c.dec_seq_lens.tolist() == [17, 64, 100, 255]
    assert (c.num_q_heads, c.num_kv_heads, c.head_dim) == (16, 8, 128)
    assert c.sm_scale == pytest.approx(1 / math.sqrt(128))
    # new-token slot = last table entry of the request; all slots distinct
    for r in range(4):
        row = c.dec_req_rows[r]
        assert c.out_loc[r] == c.page_table[row, c.dec_seq_lens[r] - 1]
    used = np.concatenate([c.page_table[c.dec_req_rows[r], :c.dec_seq_lens[r]] for r in range(4)])
    assert len(np.unique(used)) == used.size == 436
    again = W.config_c1()
    assert np.array_equal(again.k_pool, c.k_pool) and np.array_equal(again.page_table, c.page_table)


def test_small_page16_rows_are_page_contiguous_and_shared():
    c = W.small_decode(3, 4, 2, [40, 33, 64, 17], page_size=16, num_slots=4096,
                       shared_prefix=16, shared_by=(0, 1, 2, 3))
    rows = [c.page_table[c.dec_req_rows[r], :c.dec_seq_lens[r]] for r in range(4)]
    for row in rows:
        j = np.arange(row.size)
        assert np.array_equal(row, row[j - j % 16] + j % 16)
        assert row[0] % 16 == 0
        assert np.array_equal(row[:16], rows[0][:16])
    own = np.concatenate([r[16:] for r in rows])
    assert len(np.unique(own)) == own.size


def test_extend_inputs_store_the_chunk_slots():
    c = W.small_extend(4, 4, 2, [(10, 6), (0, 3)], num_slots=256, decode_lens=[5])
    assert c.ext_q.shape == (9, 4, 128) and c.ext_q_offsets.tolist() == [0, 6, 9]
    r0 = c.page_table[c.ext_req_rows[0]]
    r1 = c.page_table[c.ext_req_rows[1]]
    rd = c.page_table[c.dec_req_rows[0]]
    assert c.out_loc.tolist() == r0[10:16].tolist() + r1[0:3].tolist() + [rd[4]]


def test_causal_pair_count_closed_form_against_brute_force():
    P = [0, 7, 100]
    E = [5, 1, 33]
    brute = sum(1 for p, e in zip(P, E) for i in range(e) for j in range(p + e) if j <= p + i)
    assert metrics.causal_pairs(P, E) == brute
    assert metrics.extend_flops(P, E, 32, 128) == 4 * 32 * 128 * brute


def test_decode_bytes_count_shared_rows_once():
    c = W.small_decode(5, 4, 2, [20, 30], num_slots=256, shared_prefix=10, shared_by=(0, 1))
    kv = metrics.decode_kv_bytes(c.page_table, c.dec_req_rows, c.dec_seq_lens, 2, 128)
    assert kv == (20 + 30 - 10) * 2 * 2 * 128 * 2
    total = metrics.decode_bytes(c.page_table, c.dec_req_rows, c.dec_seq_lens, 4, 2, 128)
    assert total == kv + 4 * 50 + 2 * 2 * 4 * 128 * 2 + 4 * 2 * 4


def test_c4_length_recipe():
    rng = np.random.Generator(np.random.PCG64(4))
    L = W.synth.c4_lengths(rng)
    assert L.size == 256 and L.min() >= 1024 and L.max() <= 32768
    assert 1500 < np.median(L) < 2800
