"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case takes the oracle's source text, plants one plausible slip, loads
the result as a throw-away module and runs the independent checks of
``test_oracle_pins.py`` against it (brute force, torch SDPA, closed forms).
A mutant that passes every check would mean the pins cannot see that slip.
"""

import importlib.util
import math
import os
import types

import numpy as np
import pytest

from workloads import small_decode, small_extend
from tests.brute import brute_attention, bits_to_float, decode_brute, sdpa_extend

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")


def load_mutant(old: str, new: str) -> types.ModuleType:
    text = open(SRC).read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
    text = text.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def check_decode_brute(orc) -> bool:
    inp = small_decode(31, 4, 2, [5, 1, 9], head_dim=16, num_slots=64)
    o, l = orc.paged_decode(inp.dec_q, inp.k_pool, inp.v_pool, inp.page_table,
                            inp.dec_req_rows, inp.dec_seq_lens, inp.sm_scale, 2)
    ob, lb = decode_brute(inp)
    return np.allclose(o, ob, rtol=1e-10, atol=1e-10) and np.allclose(l, lb, rtol=1e-10, atol=1e-10)


def check_extend_sdpa(orc) -> bool:
    inp = small_extend(32, 8, 2, [(0, 9), (13, 5)], head_dim=16, num_slots=128)
    k, v = orc.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    o, _ = orc.paged_extend(inp.ext_q, k, v, inp.page_table, inp.ext_req_rows,
                            inp.ext_prefix_lens, inp.ext_extend_lens, inp.ext_q_offsets,
                            inp.sm_scale, 2)
    ok = True
    for r in range(2):
        row = inp.ext_req_rows[r]
        P, E, base = inp.ext_prefix_lens[r], inp.ext_extend_lens[r], inp.ext_q_offsets[r]
        slots = inp.page_table[row, :P + E]
        up = lambda b: ((b.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
        ref = sdpa_extend(up(inp.ext_q[base:base + E]), up(k[slots]), up(v[slots]),
                          prefix=int(P), scale=inp.sm_scale)
        ok &= np.allclose(o[base:base + E], ref, rtol=1e-9, atol=1e-11)
    return bool(ok)


def check_extend_lse_brute(orc) -> bool:
    """Every extend row's lse against the pure-Python brute force over its
    visible keys (prefix plus the new tokens up to its own)."""
    inp = small_extend(34, 4, 2, [(3, 4), (0, 3)], head_dim=8, num_slots=64)
    k, v = orc.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    _, lse = orc.paged_extend(inp.ext_q, k, v, inp.page_table, inp.ext_req_rows,
                              inp.ext_prefix_lens, inp.ext_extend_lens, inp.ext_q_offsets,
                              inp.sm_scale, 2)
    Hq = inp.ext_q.shape[1]
    ratio = Hq // 2
    for r in range(len(inp.ext_prefix_lens)):
        row = int(inp.ext_req_rows[r])
        P, E, base = (int(inp.ext_prefix_lens[r]), int(inp.ext_extend_lens[r]),
                      int(inp.ext_q_offsets[r]))
        for ii in range(E):
            slots = [int(inp.page_table[row, j]) for j in range(P + ii + 1)]
            for h in range(Hq):
                g = h // ratio
                qv = [bits_to_float(x) for x in inp.ext_q[base + ii, h]]
                ks = [[bits_to_float(x) for x in k[sl, g]] for sl in slots]
                vs = [[bits_to_float(x) for x in v[sl, g]] for sl in slots]
                _, lb = brute_attention(qv, ks, vs, inp.sm_scale)
                if abs(lse[base + ii, h] - lb) > 1e-10:
                    return False
    return True


def check_split_merge(orc) -> bool:
    inp = small_decode(33, 4, 2, [50, 17, 3], num_slots=256)
    o, l = orc.paged_decode(inp.dec_q, inp.k_pool, inp.v_pool, inp.page_table,
                            inp.dec_req_rows, inp.dec_seq_lens, inp.sm_scale, 2)
    o2, l2, _, _ = orc.paged_decode_split(inp.dec_q, inp.k_pool, inp.v_pool, inp.page_table,
                                          inp.dec_req_rows, inp.dec_seq_lens, inp.sm_scale, 2, 8)
    return np.allclose(o, o2, rtol=1e-10, atol=1e-12) and np.allclose(l, l2, rtol=1e-10, atol=1e-12)


def check_merge_closed_form(orc) -> bool:
    o = np.array([[[1.0, 2.0]], [[3.0, -4.0]]])
    out, lse = orc.merge_states(o, np.array([[0.0], [math.log(3.0)]]))
    return np.allclose(out, [[2.5, -2.5]], rtol=1e-14) and abs(lse[0] - math.log(4.0)) < 1e-14


def check_store(orc) -> bool:
    k = np.arange(8, dtype=np.uint16).reshape(4, 1, 2)
    v = (100 + np.arange(8, dtype=np.uint16)).reshape(4, 1, 2)
    kn = np.array([[[900, 901]], [[910, 911]]], np.uint16)
    vn = np.array([[[800, 801]], [[810, 811]]], np.uint16)
    ko, vo = orc.store_kv(k, v, kn, vn, np.array([3, 1]))
    return ko.reshape(-1).tolist() == [0, 1, 910, 911, 4, 5, 900, 901] and \
        vo.reshape(-1).tolist() == [100, 101, 810, 811, 104, 105, 800, 801]


ALL_CHECKS = [check_decode_brute, check_extend_sdpa, check_extend_lse_brute, check_split_merge,
              check_merge_closed_form, check_store]

MUTANTS = {
    "dropped scale": ("s = sm_scale * (keys @ q)", "s = (keys @ q)"),
    "exp without max shift in lse": ("lse = m + math.log(denom)", "lse = math.log(denom)"),
    "gqa head map modulo": ("for h in range(g * ratio, (g + 1) * ratio):\n                out[r, h]",
                            "for h in [x for x in range(Hq) if x % num_kv_heads == g]:\n                out[r, h]"),
    "table walk off by one": ("slots = [int(page_table_row[j]) for j in range(begin, end)]",
                              "slots = [int(page_table_row[j + 1]) for j in range(begin, end)]"),
    "causal mask excludes the diagonal": ("visible = P + ii + 1", "visible = P + ii"),
    "causal mask ignores the prefix": ("visible = P + ii + 1", "visible = ii + 1"),
    "merge plain average": ("w = [math.exp(x - M) for x in lses]", "w = [1.0 for x in lses]"),
    "merge lse forgets the max": ("lse[idx] = M + math.log(total)", "lse[idx] = math.log(total)"),
    "store swaps k and v": ("k_out[slot] = k_new[i]", "k_out[slot] = v_new[i]"),
    "value rows from the key pool": ("vals = gather_rows(v_pool, page_table[row], b, e, g)",
                                     "vals = gather_rows(k_pool, page_table[row], b, e, g)"),
    "extend reads q of the wrong request": ("s = sm_scale * (qf[base + ii, h, :] @ keys.T)",
                                            "s = sm_scale * (qf[ii, h, :] @ keys.T)"),
    "decode output not normalised": ("out = (p @ values) / denom", "out = (p @ values)"),
    "extend output not normalised": ("out[base + ii, h, :] = (p @ vals) / denom",
                                     "out[base + ii, h, :] = (p @ vals)"),
    "decode lse in base 2": ("lse = m + math.log(denom)", "lse = m + math.log2(denom)"),
    "extend lse in base 2": ("lse[base + ii, h] = m[:, 0] + np.log(denom[:, 0])",
                             "lse[base + ii, h] = m[:, 0] + np.log2(denom[:, 0])"),
    "split chunks drop their last key": ("e = [min((c + 1) * split_tokens, x) for x in L]",
                                         "e = [min((c + 1) * split_tokens - 1, x) for x in L]"),
}


def test_unmutated_oracle_passes_every_check():
    orc = load_mutant("import math", "import math")
    assert all(chk(orc) for chk in ALL_CHECKS)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    orc = load_mutant(old, new)
    results = {}
    for chk in ALL_CHECKS:
        try:
            results[chk.__name__] = chk(orc)
        except Exception:
            results[chk.__name__] = False
    assert not all(results.values()), f"mutant '{name}' survived: {results}"
