"""Pins of the CPU oracle against things other than itself (CPU only).

Each test fixes one part of the oracle with a closed form, an invariant,
brute force, an independent library routine (torch SDPA in float64) or a
number the source pages print.  Together they are chosen so that a
plausible slip anywhere in the oracle (dropped scale, wrong GQA head map,
off-by-one causal offset, wrong merge weights, wrong table walk) fails at
least one; ``test_oracle_mutants.py`` plants such slips and checks it.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import small_decode, small_extend, random_bf16, f32_to_bf16_bits
from tests.brute import decode_brute, sdpa_extend, bits_to_float

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# number format
# ---------------------------------------------------------------------------

def test_bf16_upcast_known_bits():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x3E00], np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, math.inf, -math.inf, 0.0, -0.0, 0.125]
    got = oracle.bf16_to_f64(bits)
    for g, w in zip(got, want):
        assert g == w
    assert math.copysign(1.0, got[6]) == -1.0


def test_bf16_round_to_nearest_even():
    one = 1.0
    cases = {
        one: 0x3F80,
        one + 2 ** -8: 0x3F80,          # halfway 1.0 / 1.0078125 -> even (1.0)
        one + 3 * 2 ** -8: 0x3F82,      # halfway 1.0078125 / 1.015625 -> even
        one + 2 ** -8 + 2 ** -30: 0x3F81,
        -2.5: 0xC020,
        3.0e38: 0x7F62,
        2.0 ** -133: 0x0001,
        2.0 ** -134: 0x0000,            # halfway 0 / min subnormal -> even (0)
        3 * 2.0 ** -134: 0x0002,        # halfway 1 / 2 ulps -> even (2)
        1e39: 0x7F80,                   # overflows to inf
    }
    got = oracle.f64_to_bf16_rne(np.array(list(cases.keys())))
    assert [int(x) for x in got] == list(cases.values())


def test_bf16_rne_matches_bit_trick_on_float32_values():
    # the generator's float32 bit trick and the oracle's float64 rounding are
    # two separate implementations of the same rule
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(4000) * np.exp(rng.uniform(-30, 30, 4000))).astype(np.float32)
    assert np.array_equal(oracle.f64_to_bf16_rne(x.astype(np.float64)), f32_to_bf16_bits(x))


# ---------------------------------------------------------------------------
# a1 store_kv
# ---------------------------------------------------------------------------

def test_store_kv_hand_example():
    k = np.arange(4 * 1 * 2, dtype=np.uint16).reshape(4, 1, 2)          # slots 0..3
    v = (100 + np.arange(8, dtype=np.uint16)).reshape(4, 1, 2)
    kn = np.array([[[900, 901]], [[910, 911]]], np.uint16)
    vn = np.array([[[800, 801]], [[810, 811]]], np.uint16)
    ko, vo = oracle.store_kv(k, v, kn, vn, np.array([3, 1]))
    assert ko.reshape(-1).tolist() == [0, 1, 910, 911, 4, 5, 900, 901]
    assert vo.reshape(-1).tolist() == [100, 101, 810, 811, 104, 105, 800, 801]
    assert k.reshape(-1).tolist() == list(range(8))        # inputs untouched


def test_store_kv_int32_and_int64_indices_agree():
    rng = np.random.default_rng(3)
    k = random_bf16(rng, (64, 2, 8)); v = random_bf16(rng, (64, 2, 8))
    kn = random_bf16(rng, (5, 2, 8)); vn = random_bf16(rng, (5, 2, 8))
    loc = rng.permutation(64)[:5]
    a = oracle.store_kv(k, v, kn, vn, loc.astype(np.int32))
    b = oracle.store_kv(k, v, kn, vn, loc.astype(np.int64))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    untouched = np.setdiff1d(np.arange(64), loc)
    assert np.array_equal(a[0][untouched], k[untouched])
    assert np.array_equal(a[0][loc], kn)


# ---------------------------------------------------------------------------
# a4 decode: brute force, SDPA, closed forms, invariants
# ---------------------------------------------------------------------------

def _stored(inp):
    return oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)


def _decode(inp, k=None, v=None, **kw):
    if k is None:
        k, v = _stored(inp)
    return oracle.paged_decode(inp.dec_q, k, v, inp.page_table, inp.dec_req_rows,
                               inp.dec_seq_lens, kw.get("sm_scale", inp.sm_scale),
                               inp.num_kv_heads)


def test_decode_matches_pure_python_brute_force():
    inp = small_decode(11, 4, 2, [5, 1, 9], head_dim=16, num_slots=64)
    o, l = _decode(inp, inp.k_pool, inp.v_pool)
    ob, lb = decode_brute(inp)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l, lb, rtol=1e-12, atol=1e-12)


def test_decode_matches_torch_sdpa_float64():
    inp = small_decode(12, 8, 2, [33, 7, 70], head_dim=32, num_slots=256)
    k, v = _stored(inp)
    o, _ = _decode(inp, k, v)
    for r in range(inp.num_decode):
        row = inp.dec_req_rows[r]
        L = inp.dec_seq_lens[r]
        slots = inp.page_table[row, :L]
        kk = oracle.bf16_to_f64(k[slots]); vv = oracle.bf16_to_f64(v[slots])
        q = oracle.bf16_to_f64(inp.dec_q[r:r + 1])
        ref = sdpa_extend(q, kk, vv, prefix=L - 1, scale=inp.sm_scale)[0]
        np.testing.assert_allclose(o[r], ref, rtol=1e-10, atol=1e-12)


def test_seq_len_one_returns_the_value_row_exactly():
    inp = small_decode(13, 4, 4, [1, 1], num_slots=32)
    k, v = _stored(inp)
    o, l = _decode(inp, k, v)
    for r in range(2):
        slot = inp.page_table[inp.dec_req_rows[r], 0]
        for h in range(4):
            assert np.array_equal(o[r, h], oracle.bf16_to_f64(v[slot, h]))
            s0 = inp.sm_scale * sum(bits_to_float(a) * bits_to_float(b)
                                    for a, b in zip(inp.dec_q[r, h], k[slot, h]))
            assert l[r, h] == pytest.approx(s0, rel=1e-12, abs=1e-12)


def test_zero_scale_gives_mean_of_values_and_log_length():
    inp = small_decode(14, 4, 2, [6, 11], num_slots=64)
    k, v = _stored(inp)
    o, l = _decode(inp, k, v, sm_scale=0.0)
    for r in range(2):
        L = inp.dec_seq_lens[r]
        slots = inp.page_table[inp.dec_req_rows[r], :L]
        for h in range(4):
            want = oracle.bf16_to_f64(v[slots, h // 2]).mean(axis=0)
            np.testing.assert_allclose(o[r, h], want, rtol=1e-13, atol=1e-13)
            assert l[r, h] == pytest.approx(math.log(L), rel=1e-14)


def test_slot_permutation_leaves_results_bitwise_unchanged():
    inp = small_decode(15, 8, 2, [40, 3, 90], num_slots=256)
    k, v = _stored(inp)
    o1, l1 = _decode(inp, k, v)
    pi = np.random.default_rng(5).permutation(inp.num_slots)
    k2 = np.empty_like(k); v2 = np.empty_like(v)
    k2[pi] = k; v2[pi] = v
    pt2 = pi[inp.page_table].astype(np.int32)
    o2, l2 = oracle.paged_decode(inp.dec_q, k2, v2, pt2, inp.dec_req_rows,
                                 inp.dec_seq_lens, inp.sm_scale, inp.num_kv_heads)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_gqa_equals_mha_on_repeated_kv_heads():
    inp = small_decode(16, 8, 2, [25, 9], num_slots=128)
    k, v = _stored(inp)
    o, l = _decode(inp, k, v)
    k_rep = np.repeat(k, 4, axis=1)       # head h of the MHA pool = kv head h // 4
    v_rep = np.repeat(v, 4, axis=1)
    om, lm = oracle.paged_decode(inp.dec_q, k_rep, v_rep, inp.page_table,
                                 inp.dec_req_rows, inp.dec_seq_lens, inp.sm_scale, 8)
    assert np.array_equal(o, om) and np.array_equal(l, lm)


def test_shared_prefix_equals_duplicated_prefix():
    inp = small_decode(17, 4, 2, [48, 64, 20], num_slots=512,
                       shared_prefix=16, shared_by=(0, 1, 2))
    k, v = _stored(inp)
    o1, l1 = _decode(inp, k, v)
    # copy the shared 16 slots of requests 1 and 2 to fresh, unused slots
    pt = inp.page_table.copy()
    used = set()
    for r in range(3):
        used.update(pt[inp.dec_req_rows[r], :inp.dec_seq_lens[r]].tolist())
    free = [s for s in range(inp.num_slots) if s not in used]
    k2, v2 = k.copy(), v.copy()
    for r in (1, 2):
        row = inp.dec_req_rows[r]
        for j in range(16):
            dst = free.pop()
            k2[dst] = k[pt[row, j]]; v2[dst] = v[pt[row, j]]
            pt[row, j] = dst
    o2, l2 = oracle.paged_decode(inp.dec_q, k2, v2, pt, inp.dec_req_rows,
                                 inp.dec_seq_lens, inp.sm_scale, inp.num_kv_heads)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_size_16_table_gives_identical_results_to_its_token_view():
    inp = small_decode(18, 4, 2, [37, 16, 50], page_size=16, num_slots=1024)
    # the table is token granular and page-contiguous: check the layout rule,
    # then rebuild each row from its page ids and compare results
    pt2 = inp.page_table.copy()
    for r in range(3):
        row = inp.dec_req_rows[r]; L = inp.dec_seq_lens[r]
        pages = oracle.token_table_to_page_ids(inp.page_table[row], L, 16)
        rebuilt = oracle.page_ids_to_token_table(pages, L, 16)
        assert np.array_equal(rebuilt, inp.page_table[row, :L])
        pt2[row, :L] = rebuilt
    k, v = _stored(inp)
    o1, l1 = _decode(inp, k, v)
    o2, l2 = oracle.paged_decode(inp.dec_q, k, v, pt2, inp.dec_req_rows,
                                 inp.dec_seq_lens, inp.sm_scale, inp.num_kv_heads)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_table_view_golden():
    with open(os.path.join(GOLDEN, "page_table_view.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        got = oracle.token_table_to_page_ids(np.array(c["token_row"]), c["length"], c["page_size"])
        assert got.tolist() == c["expected_page_ids"]
        back = oracle.page_ids_to_token_table(c["expected_page_ids"], c["length"], c["page_size"])
        assert back.tolist() == c["token_row"]


# ---------------------------------------------------------------------------
# a5 merge
# ---------------------------------------------------------------------------

def test_merge_closed_forms():
    o = np.array([[[1.0, 2.0]], [[3.0, -4.0]]])        # S=2, N=1, D=2
    # equal lse: plain average, lse + ln 2
    out, lse = oracle.merge_states(o, np.array([[0.5], [0.5]]))
    assert out.tolist() == [[2.0, -1.0]] and lse[0] == pytest.approx(0.5 + math.log(2), abs=1e-15)
    # an empty part carries no weight
    out, lse = oracle.merge_states(o, np.array([[-math.inf], [1.25]]))
    assert out.tolist() == [[3.0, -4.0]] and lse[0] == 1.25
    # all empty -> zeros, -inf
    out, lse = oracle.merge_states(o, np.array([[-math.inf], [-math.inf]]))
    assert out.tolist() == [[0.0, 0.0]] and lse[0] == -math.inf
    # weights e^{lse}: lse = (0, ln 3) -> weights 1:3
    out, lse = oracle.merge_states(o, np.array([[0.0], [math.log(3.0)]]))
    np.testing.assert_allclose(out, [[(1 + 9) / 4, (2 - 12) / 4]], rtol=1e-15)
    assert lse[0] == pytest.approx(math.log(4.0), rel=1e-15)


@pytest.mark.parametrize("split", [1, 7, 16, 64, 1000])
def test_split_then_merge_equals_unsplit(split):
    inp = small_decode(19, 8, 2, [100, 17, 64, 1], num_slots=512)
    k, v = _stored(inp)
    o, l = _decode(inp, k, v)
    o2, l2, po, pl = oracle.paged_decode_split(inp.dec_q, k, v, inp.page_table,
                                               inp.dec_req_rows, inp.dec_seq_lens,
                                               inp.sm_scale, inp.num_kv_heads, split)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l, rtol=1e-13, atol=1e-13)


def test_empty_request_is_zero_with_minus_inf_lse():
    o, l = oracle.attend_one(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.3)
    assert o.tolist() == [0.0] * 4 and l == -math.inf


# ---------------------------------------------------------------------------
# a6 extend
# ---------------------------------------------------------------------------

def _stored_ext(inp):
    return oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)


def _extend(inp, k, v, **kw):
    return oracle.paged_extend(inp.ext_q, k, v, inp.page_table, inp.ext_req_rows,
                               inp.ext_prefix_lens, inp.ext_extend_lens, inp.ext_q_offsets,
                               inp.sm_scale, inp.num_kv_heads, **kw)


def test_extend_matches_torch_sdpa_with_prefix():
    inp = small_extend(21, 8, 2, [(0, 9), (13, 5), (40, 17)], head_dim=32, num_slots=256)
    k, v = _stored_ext(inp)
    o, _ = _extend(inp, k, v)
    for r in range(3):
        row = inp.ext_req_rows[r]
        P, E, base = inp.ext_prefix_lens[r], inp.ext_extend_lens[r], inp.ext_q_offsets[r]
        slots = inp.page_table[row, :P + E]
        ref = sdpa_extend(oracle.bf16_to_f64(inp.ext_q[base:base + E]),
                          oracle.bf16_to_f64(k[slots]), oracle.bf16_to_f64(v[slots]),
                          prefix=int(P), scale=inp.sm_scale)
        np.testing.assert_allclose(o[base:base + E], ref, rtol=1e-10, atol=1e-12)


def test_extend_without_prefix_matches_torch_is_causal():
    import torch
    inp = small_extend(22, 4, 4, [(0, 12)], head_dim=16, num_slots=64)
    k, v = _stored_ext(inp)
    o, _ = _extend(inp, k, v)
    slots = inp.page_table[inp.ext_req_rows[0], :12]
    q = torch.from_numpy(oracle.bf16_to_f64(inp.ext_q).transpose(1, 0, 2).copy())
    kk = torch.from_numpy(oracle.bf16_to_f64(k[slots]).transpose(1, 0, 2).copy())
    vv = torch.from_numpy(oracle.bf16_to_f64(v[slots]).transpose(1, 0, 2).copy())
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True,
                                                           scale=inp.sm_scale)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_chunked_extend_equals_one_full_prefill():
    N = 45
    full = small_extend(23, 4, 2, [(0, N)], num_slots=128)
    k, v = _stored_ext(full)
    of, lf = _extend(full, k, v)
    row = full.page_table[full.ext_req_rows[0]]
    # same keys in the pool, now processed as chunks 0..12, 12..30, 30..45
    cuts = [0, 12, 30, N]
    for a, b in zip(cuts[:-1], cuts[1:]):
        oc, lc = oracle.paged_extend(full.ext_q[a:b], k, v, row[None, :],
                                     np.array([0]), np.array([a]), np.array([b - a]),
                                     np.array([0, b - a]), full.sm_scale, 2)
        np.testing.assert_allclose(oc, of[a:b], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lc, lf[a:b], rtol=1e-13, atol=1e-13)


def test_decode_equals_extend_of_one_token():
    inp = small_decode(24, 8, 2, [30, 1, 77], num_slots=256)
    k, v = _stored(inp)
    od, ld = _decode(inp, k, v)
    L = inp.dec_seq_lens
    oe, le = oracle.paged_extend(inp.dec_q, k, v, inp.page_table, inp.dec_req_rows,
                                 L - 1, np.ones_like(L), np.arange(len(L) + 1),
                                 inp.sm_scale, inp.num_kv_heads)
    np.testing.assert_allclose(oe, od, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(le, ld, rtol=1e-13, atol=1e-14)


def test_extend_first_query_without_prefix_is_its_own_value_row():
    inp = small_extend(25, 4, 2, [(0, 5)], num_slots=64)
    k, v = _stored_ext(inp)
    o, _ = _extend(inp, k, v)
    slot0 = inp.page_table[inp.ext_req_rows[0], 0]
    for h in range(4):
        assert np.array_equal(o[0, h], oracle.bf16_to_f64(v[slot0, h // 2]))


def test_extend_query_subset_matches_full():
    inp = small_extend(26, 4, 2, [(8, 20), (0, 7)], num_slots=128)
    k, v = _stored_ext(inp)
    o, l = _extend(inp, k, v)
    sub = [0, 5, 19, 21, 26]
    o2, l2 = _extend(inp, k, v, query_subset=sub, block_rows=2)
    np.testing.assert_allclose(o2[sub], o[sub], rtol=1e-13, atol=1e-14)
    rest = [i for i in range(27) if i not in sub]
    assert np.all(o2[rest] == 0) and np.all(l2[rest] == -np.inf)


# ---------------------------------------------------------------------------
# the pages' printed arithmetic
# ---------------------------------------------------------------------------

def test_pages_kv_arithmetic_golden():
    with open(os.path.join(GOLDEN, "pages_kv_arithmetic.json")) as f:
        g = json.load(f)
    t = g["kv_bytes_per_token"]
    per_tok = oracle.kv_bytes_per_token(t["num_layers"], t["num_kv_heads"], t["head_dim"], t["dtype_bytes"])
    assert per_tok == t["expected_bytes"] == 128 * 1024
    assert g["request_4k"]["tokens"] * per_tok == g["request_4k"]["expected_bytes"]
    c = g["concurrent_100x4k"]
    assert c["requests"] * c["tokens"] * per_tok == c["expected_gib"] * 2 ** 30
    b1 = g["h100_budget_page1"]
    page1 = oracle.kv_bytes_per_page(32, b1["page_size"], 8, 128, 2)
    assert oracle.pool_pages_for_budget(b1["budget_gib"] * 2 ** 30, page1) == b1["expected_pages"]
    b64 = g["h100_budget_page64"]
    page64 = oracle.kv_bytes_per_page(32, b64["page_size"], 8, 128, 2)
    assert page64 == b64["expected_page_bytes"]
    n = oracle.pool_pages_for_budget(b64["budget_gib"] * 2 ** 30, page64)
    assert n == b64["expected_pages"] and n * 64 == b64["expected_tokens"]
    a = g["available_budget"]
    assert a["init_free_gib"] - a["post_free_gib"] == a["expected_model_gib"]
    assert math.floor(a["memory_ratio"] * a["init_free_gib"] - a["expected_model_gib"]) == a["expected_available_gib_floor"]
