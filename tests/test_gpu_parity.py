"""GPU parity of the HIP kernels against the fp64 CPU oracle (small shapes).

Sizes are chosen so the oracle finishes in seconds while the kernels still
see several tiles, a ragged tail and the edge cases (one key, exact tile
multiples, empty work).  Bars: store_kv and indexing invariants bit-exact;
attention within max abs 2e-2 and max abs / max |ref| 1e-2.
"""

import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_30_amd as msgl
from workloads import small_decode, small_extend, random_bf16, config_c1, f32_to_bf16_bits
from tests.gpu_util import (Uploaded, up, bits, f64, assert_close, assert_lse_close)

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def oracle_pool(inp):
    return oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)


def oracle_decode(inp, kp, vp):
    return oracle.paged_decode(inp.dec_q, kp, vp, inp.page_table, inp.dec_req_rows,
                               inp.dec_seq_lens, inp.sm_scale, inp.num_kv_heads)


def oracle_extend(inp, kp, vp):
    return oracle.paged_extend(inp.ext_q, kp, vp, inp.page_table, inp.ext_req_rows,
                               inp.ext_prefix_lens, inp.ext_extend_lens, inp.ext_q_offsets,
                               inp.sm_scale, inp.num_kv_heads)


# ---------------------------------------------------------------------------
# store_kv
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("index_dtype", [np.int32, np.int64])
def test_store_kv_bit_exact_c1(index_dtype):
    banner(f"store_kv C1 index {index_dtype.__name__}")
    inp = config_c1()
    u = Uploaded(inp)
    u.out_loc = up(inp.out_loc.astype(index_dtype))
    u.store()
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    assert np.array_equal(bits(u.k), kp) and np.array_equal(bits(u.v), vp)


@pytest.mark.parametrize("n", [1, 3, 257, 4000])
def test_store_kv_strided_rows_and_ragged_counts(n):
    banner(f"store_kv strided n={n}")
    rng = np.random.default_rng(n)
    slots, hkv, d = 8192, 8, 128
    k = random_bf16(rng, (slots, hkv, d)); v = random_bf16(rng, (slots, hkv, d))
    # new rows as views into a wider [n, 3, Hkv, D] buffer (as a fused qkv split would give)
    fused = random_bf16(rng, (n, 3, hkv, d))
    loc = rng.permutation(slots)[:n].astype(np.int64)
    kg, vg = up(k), up(v)
    fg = up(fused)
    msgl.store_kv(kg, vg, fg[:, 1], fg[:, 2], up(loc))
    torch.cuda.synchronize()
    kp, vp = oracle.store_kv(k, v, fused[:, 1], fused[:, 2], loc)
    assert np.array_equal(bits(kg), kp) and np.array_equal(bits(vg), vp)


def test_store_kv_fp32_and_narrow_rows():
    banner("store_kv fp32 / odd row size")
    rng = np.random.default_rng(5)
    k = rng.standard_normal((300, 3, 6)).astype(np.float32)   # 72-byte rows -> 8-byte units
    v = rng.standard_normal((300, 3, 6)).astype(np.float32)
    kn = rng.standard_normal((17, 3, 6)).astype(np.float32)
    vn = rng.standard_normal((17, 3, 6)).astype(np.float32)
    loc = rng.permutation(300)[:17].astype(np.int32)
    kg, vg = up(k), up(v)
    msgl.store_kv(kg, vg, up(kn), up(vn), up(loc))
    torch.cuda.synchronize()
    kp, vp = oracle.store_kv(k, v, kn, vn, loc)
    assert np.array_equal(kg.cpu().numpy(), kp) and np.array_equal(vg.cpu().numpy(), vp)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def test_decode_c1_full():
    banner("decode C1")
    inp = config_c1()
    u = Uploaded(inp)
    u.store()
    out, lse = u.decode()
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(out, ro, "C1 out")
    assert_lse_close(lse, rl, "C1 lse")


DECODE_CASES = [
    # (hq, hkv, seq_lens, split_tokens)
    (8, 8, [1, 31, 32, 33], 0),
    (16, 8, [64, 65, 255, 256, 257, 600], 0),
    (32, 8, [700, 1, 129, 1024, 513], 64),
    (32, 8, [700, 1, 129, 1024, 513], 96),
    (64, 8, [1500, 2048, 3, 777], 256),
    (16, 1, [300, 45], 32),
    (32, 2, [90, 1000, 1001], 128),
    (4, 2, [5, 40], 0),
    # more kv heads than one workgroup takes (16 and 32: two and four groups
    # of 8), and 4 kv heads
    (16, 16, [700, 1, 129, 2000], 0),
    (16, 16, [700, 1, 129, 2000], 128),
    (32, 32, [300, 1025, 64], 0),
    (8, 4, [1, 500, 33], 0),
    (64, 4, [1200, 7], 64),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_parity(case):
    hq, hkv, lens, split = DECODE_CASES[case]
    banner(f"decode hq={hq} hkv={hkv} lens={lens} split={split}")
    inp = small_decode(40 + case, hq, hkv, lens, num_slots=8192)
    u = Uploaded(inp)
    u.store()
    out, lse = u.decode(split_tokens=split)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(out, ro, f"decode case {case}")
    assert_lse_close(lse, rl, f"decode case {case}")


def test_decode_without_req_rows_and_strided_q():
    banner("decode identity rows + strided q")
    inp = small_decode(60, 32, 8, [100, 300, 2], num_slots=2048)
    # table rows in request order; q as a view into a wider buffer
    pt = np.stack([inp.page_table[r] for r in inp.dec_req_rows] + [inp.page_table[-1]])
    u = Uploaded(inp)
    u.store()
    wide = torch.zeros((3, 48, 128), dtype=torch.bfloat16, device="cuda")
    wide[:, 8:40] = u.dq
    q = wide[:, 8:40]
    out, lse = msgl.paged_decode(q, u.k, u.v, up(pt.astype(np.int32)), u.d_lens, u.d_max,
                                 inp.sm_scale, split_tokens=64)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(out, ro, "identity rows")


def test_decode_seq_len_one_is_the_value_row_bit_exact():
    banner("decode seq_len=1 bitwise")
    inp = small_decode(61, 32, 8, [1] * 7, num_slots=512)
    u = Uploaded(inp)
    u.store()
    out, lse = u.decode()
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    got = bits(out)
    for r in range(7):
        slot = inp.page_table[inp.dec_req_rows[r], 0]
        for h in range(32):
            assert np.array_equal(got[r, h], vp[slot, h // 4]), (r, h)


def test_decode_slot_permutation_bitwise():
    banner("decode slot permutation bitwise")
    inp = small_decode(62, 32, 8, [700, 33, 1200, 64], num_slots=4096)
    u = Uploaded(inp)
    u.store()
    o1, l1 = u.decode(split_tokens=256)
    pi = np.random.default_rng(9).permutation(inp.num_slots)
    kp, vp = oracle_pool(inp)
    k2 = np.empty_like(kp); v2 = np.empty_like(vp)
    k2[pi] = kp; v2[pi] = vp
    pt2 = pi[inp.page_table].astype(np.int32)
    o2, l2 = msgl.paged_decode(u.dq, up(k2), up(v2), up(pt2), u.d_lens, u.d_max, inp.sm_scale,
                               req_rows=u.d_rows, split_tokens=256)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())


def test_decode_page_size_16_matches_page_size_1_bitwise_and_oracle():
    banner("decode page_size 16 vs 1")
    inp = small_decode(63, 32, 8, [1000, 17, 512, 300], page_size=16, num_slots=8192,
                       shared_prefix=16, shared_by=(0, 1, 2, 3))
    u = Uploaded(inp)
    u.store()
    o16, l16 = u.decode(page_size=16)
    o1, l1 = u.decode(page_size=1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o16), bits(o1))
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(o16, ro, "page16")


def test_decode_is_deterministic():
    banner("decode determinism")
    inp = small_decode(64, 64, 8, [3000, 5, 1800], num_slots=8192)
    u = Uploaded(inp)
    u.store()
    outs = [bits(u.decode()[0]) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_decode_empty_request():
    banner("decode empty request")
    inp = small_decode(65, 16, 8, [40, 1, 70], num_slots=1024)
    u = Uploaded(inp)
    u.store()
    lens = inp.dec_seq_lens.copy()
    lens[1] = 0
    out, lse = msgl.paged_decode(u.dq, u.k, u.v, u.pt, up(lens), u.d_max, inp.sm_scale,
                                 req_rows=u.d_rows, split_tokens=32)
    torch.cuda.synchronize()
    assert np.all(f64(out)[1] == 0) and np.all(np.isneginf(lse.cpu().numpy()[1]))
    kp, vp = oracle_pool(inp)
    ro, _ = oracle.paged_decode(inp.dec_q, kp, vp, inp.page_table, inp.dec_req_rows, lens,
                                inp.sm_scale, inp.num_kv_heads)
    assert_close(out, ro, "empty request batch")


@pytest.mark.parametrize("lens_kind", ["tiny", "zeros_at_edges", "many"])
def test_decode_balanced_ranges_edge_cases(lens_kind):
    """Balanced mode: fewer keys than workgroups, empty requests, >64 requests."""
    banner(f"decode balanced {lens_kind}")
    rng = np.random.default_rng(7)
    if lens_kind == "tiny":
        lens = rng.integers(1, 4, 300)                   # T ~ 600 keys
    elif lens_kind == "zeros_at_edges":
        lens = rng.integers(1, 900, 70)
        lens[0] = lens[33] = lens[-1] = lens[-2] = 0
    else:
        lens = rng.integers(1, 2000, 200)
    lens = lens.astype(np.int64)
    gen_lens = np.maximum(lens, 1)                       # generator needs >= 1 key
    inp = small_decode(67, 32, 8, gen_lens, num_slots=1 << 19)
    u = Uploaded(inp)
    u.store()
    lens32 = lens.astype(np.int32)
    out, lse = msgl.paged_decode(u.dq, u.k, u.v, u.pt, up(lens32), u.d_max, inp.sm_scale,
                                 req_rows=u.d_rows)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    sample = np.unique(np.concatenate([np.where(lens == 0)[0], np.arange(0, len(lens), 7),
                                       [len(lens) - 1]]))
    ro, rl = oracle.paged_decode(inp.dec_q[sample], kp, vp, inp.page_table,
                                 inp.dec_req_rows[sample], lens32[sample], inp.sm_scale,
                                 inp.num_kv_heads)
    assert_close(out[torch.from_numpy(sample).cuda()], ro, f"balanced {lens_kind}")
    assert_lse_close(lse[torch.from_numpy(sample).cuda()], rl, f"balanced {lens_kind}")


def test_decode_workspace_reused_across_shapes():
    """One workspace serves calls of different shapes in a row (its contents on
    entry are ignored)."""
    banner("decode workspace reuse")
    cases = [(32, 8, np.random.default_rng(3).integers(1, 2000, 60)),
             (16, 8, [64, 65, 255, 256, 257, 600]),
             (64, 8, [1500, 2048, 3, 777]),
             (8, 2, [900, 1, 400]),
             (32, 8, np.random.default_rng(4).integers(500, 3000, 20))]
    need = max(msgl.paged_decode_workspace_size(len(lens), hq, hkv, int(np.max(lens)))[0]
               for hq, hkv, lens in cases)
    ws = msgl.alloc_workspace(need)
    ws.fill_(0x7f)
    for k in range(2 * len(cases)):
        hq, hkv, lens = cases[k % len(cases)]
        inp = small_decode(80 + k % len(cases), hq, hkv, np.asarray(lens), num_slots=1 << 17)
        u = Uploaded(inp)
        u.store()
        out, lse = msgl.paged_decode(u.dq, u.k, u.v, u.pt, u.d_lens, u.d_max, inp.sm_scale,
                                     req_rows=u.d_rows, workspace=ws)
        torch.cuda.synchronize()
        kp, vp = oracle_pool(inp)
        sel = np.unique(np.linspace(0, len(inp.dec_seq_lens) - 1, 12).astype(int))
        ro, rl = oracle.paged_decode(inp.dec_q[sel], kp, vp, inp.page_table, inp.dec_req_rows[sel],
                                     inp.dec_seq_lens[sel], inp.sm_scale, inp.num_kv_heads)
        t = torch.from_numpy(sel).cuda()
        assert_close(out[t], ro, f"reuse call {k}")
        assert_lse_close(lse[t], rl, f"reuse call {k}")


def test_decode_zero_scale_is_mean_of_values():
    banner("decode sm_scale=0")
    inp = small_decode(66, 32, 8, [100, 37], num_slots=1024, sm_scale=0.0)
    u = Uploaded(inp)
    u.store()
    out, lse = u.decode(split_tokens=32)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    for r in range(2):
        L = inp.dec_seq_lens[r]
        slots = inp.page_table[inp.dec_req_rows[r], :L]
        want = oracle.bf16_to_f64(vp[slots]).mean(axis=0)           # [Hkv, D]
        ref = np.repeat(want, 4, axis=0)
        assert_close(out[r], ref, f"mean r={r}")
        assert np.allclose(lse.cpu().numpy()[r], math.log(L), atol=1e-5)


# ---------------------------------------------------------------------------
# merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("parts", [1, 2, 7])
def test_merge_states_parity(parts):
    banner(f"merge parts={parts}")
    rng = np.random.default_rng(parts)
    N, H, D = 9, 16, 128
    po = rng.standard_normal((parts, N, H, D)).astype(np.float32)
    pl = (rng.standard_normal((parts, N, H)) * 3).astype(np.float32)
    if parts > 1:
        pl[0, 2, :] = -np.inf               # an empty part
        pl[:, 3, 5] = -np.inf               # an all-empty (row, head)
    out, lse = msgl.merge_states(up(po), up(pl), out_dtype=torch.float32)
    outb, _ = msgl.merge_states(up(po), up(pl), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_states(po.astype(np.float64), pl.astype(np.float64))
    assert np.allclose(out.cpu().numpy(), ro, atol=1e-5, rtol=1e-5)
    assert_close(outb, ro, "merge bf16")
    got_l = lse.cpu().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.allclose(got_l[fin], rl[fin], atol=1e-5)
    if parts > 1:
        assert np.all(out.cpu().numpy()[3, 5] == 0)


# ---------------------------------------------------------------------------
# extend
# ---------------------------------------------------------------------------

EXTEND_CASES = [
    # (hq, hkv, specs)
    (32, 8, [(0, 1), (0, 33), (7, 64), (100, 65)]),
    (32, 8, [(300, 200), (0, 129), (64, 31)]),
    (8, 8, [(50, 130)]),
    (16, 8, [(0, 257), (1, 3)]),
    (64, 8, [(200, 40), (0, 77)]),
    (16, 1, [(90, 70)]),
    (16, 16, [(100, 90), (0, 40)]),
    (32, 32, [(64, 70)]),
    (8, 4, [(33, 129)]),
    (32, 2, [(5, 100), (0, 17)]),
]


@pytest.mark.parametrize("case", range(len(EXTEND_CASES)))
def test_extend_parity(case):
    hq, hkv, specs = EXTEND_CASES[case]
    banner(f"extend hq={hq} hkv={hkv} specs={specs}")
    inp = small_extend(80 + case, hq, hkv, specs, num_slots=4096)
    u = Uploaded(inp)
    u.store()
    out, lse = u.extend()
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_extend(inp, kp, vp)
    assert_close(out, ro, f"extend case {case}")
    assert_lse_close(lse, rl, f"extend case {case}")


def test_extend_planned_order_is_bitwise_the_natural_order():
    # the work-list planner only reorders workgroups; empty requests included
    banner("extend planned vs natural order")
    inp = small_extend(95, 32, 8, [(0, 0), (500, 300), (40, 0), (2000, 70), (0, 1), (129, 257)],
                       num_slots=8192)
    u = Uploaded(inp)
    u.store()
    op, lp = u.extend(plan=True)
    on, ln = u.extend(plan=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(op), bits(on))
    assert np.array_equal(lp.cpu().numpy().view(np.uint32), ln.cpu().numpy().view(np.uint32))
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_extend(inp, kp, vp)
    assert_close(op, ro, "extend planned")
    assert_lse_close(lp, rl, "extend planned lse")


def test_extend_zero_scale_is_causal_mean_of_values():
    # sm_scale = 0: every visible key weighs the same, so query i of a
    # request with prefix P gets the mean of V over keys 0 .. P + i
    banner("extend sm_scale=0")
    inp = small_extend(93, 32, 8, [(70, 90), (0, 65)], num_slots=2048, sm_scale=0.0)
    u = Uploaded(inp)
    u.store()
    out, lse = u.extend()
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    got = f64(out)
    got_lse = lse.cpu().numpy()
    for r in range(inp.num_extend):
        P, E, base = int(inp.ext_prefix_lens[r]), int(inp.ext_extend_lens[r]), int(inp.ext_q_offsets[r])
        slots = inp.page_table[inp.ext_req_rows[r], :P + E]
        vrows = oracle.bf16_to_f64(vp[slots])                       # [P+E, Hkv, D]
        cmean = np.cumsum(vrows, axis=0) / np.arange(1, P + E + 1)[:, None, None]
        for i in (0, 1, E // 2, E - 1):
            ref = np.repeat(cmean[P + i], 4, axis=0)
            assert np.abs(got[base + i] - ref).max() <= 2e-2, (r, i)
            assert np.allclose(got_lse[base + i], math.log(P + i + 1), atol=1e-4)


def test_extend_negative_scale():
    banner("extend sm_scale<0")
    inp = small_extend(94, 16, 8, [(33, 70), (0, 40)], num_slots=2048, sm_scale=-0.09)
    u = Uploaded(inp)
    u.store()
    out, lse = u.extend()
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_extend(inp, kp, vp)
    assert_close(out, ro, "extend negative scale")
    assert_lse_close(lse, rl, "extend negative scale lse")


def growing_scores(inp, sign, grow=0.2, seed=0):
    """The same batch with every request's keys rebuilt so that scaled scores
    rise by about ``grow`` log2 units per key position (q entries are shifted
    to mean 2, K rows carry sign * g * position plus noise).  Every 64-key
    tile then holds a new maximum more than 8 log2 units above the last one,
    so the online softmax has to rescale its running sum and output on every
    tile of every request, extend and decode alike."""
    rng = np.random.default_rng(seed)
    kp, _ = oracle_pool(inp)
    kf = oracle.bf16_to_f64(kp)
    c = abs(inp.sm_scale) * math.log2(math.e)
    g = grow / (c * 2.0 * inp.head_dim)
    spans = [(int(r), int(p) + int(e)) for r, p, e in
             zip(inp.ext_req_rows, inp.ext_prefix_lens, inp.ext_extend_lens)]
    spans += [(int(r), int(n)) for r, n in zip(inp.dec_req_rows, inp.dec_seq_lens)]
    for row, n in spans:
        slots = inp.page_table[row, :n]
        t = np.arange(n, dtype=np.float64)[:, None, None]
        kf[slots] = sign * g * t + 0.3 * rng.standard_normal((n,) + kf.shape[1:])
    kbits = f32_to_bf16_bits(kf.astype(np.float32))
    shift = lambda q: None if q is None else f32_to_bf16_bits(
        (oracle.bf16_to_f64(q) + 2.0).astype(np.float32))
    return dataclasses.replace(inp, k_pool=kbits, k_new=kbits[inp.out_loc],
                               ext_q=shift(inp.ext_q), dec_q=shift(inp.dec_q))


@pytest.mark.parametrize("scale", [0.0884, -0.09])
def test_scores_growing_along_keys_rescale_every_tile(scale):
    banner(f"growing scores, sm_scale={scale}")
    base = small_extend(96, 32, 8, [(130, 70), (0, 200), (64, 1)], num_slots=4096,
                        decode_lens=(150, 300, 33), sm_scale=scale)
    inp = growing_scores(base, 1.0 if scale > 0 else -1.0)
    u = Uploaded(inp)
    u.store()
    eo, el = u.extend()
    do, dl = u.decode()
    do_fixed, _ = u.decode(split_tokens=64)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_extend(inp, kp, vp)
    # the weights really are concentrated near each row's last visible key
    assert float(rl.max()) > 20.0
    assert_close(eo, ro, "extend, growing scores")
    assert_lse_close(el, rl, "extend lse, growing scores")
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(do, ro, "decode, growing scores")
    assert_close(do_fixed, ro, "decode (fixed chunks), growing scores")
    assert_lse_close(dl, rl, "decode lse, growing scores")


def test_extend_with_shared_prefix_and_page_size_16():
    banner("extend shared prefix, page 16 vs 1")
    inp = small_extend(90, 32, 8, [(64, 100), (64, 37), (128, 64)], page_size=16,
                       num_slots=8192, shared_prefix=64, shared_by=(0, 1, 2))
    u = Uploaded(inp)
    u.store()
    o16, _ = u.extend(page_size=16)
    o1, _ = u.extend(page_size=1)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o16), bits(o1))
    kp, vp = oracle_pool(inp)
    ro, _ = oracle_extend(inp, kp, vp)
    assert_close(o16, ro, "extend page16")


def test_page_size_16_reads_one_entry_per_page():
    """At page_size 16 the kernels read only each page's first column of the
    token table (the every-P-th-column view): with every other column
    overwritten by out-of-pool values, decode, fused store + decode and
    extend return the bits they return on the intact table at page_size 1.
    (A kernel that read a poisoned column would clamp it to the last slot and
    change the result; it could not leave the pool.)"""
    banner("page_size 16: one table entry per page")
    inp = small_extend(91, 32, 8, [(64, 100), (0, 77), (128, 64)], page_size=16,
                       num_slots=8192, decode_lens=[1000, 17, 512, 300, 16, 33],
                       shared_prefix=64, shared_by=(0, 2))
    u = Uploaded(inp)
    u.store()
    o1, l1 = u.decode(page_size=1)
    e1, el1 = u.extend(page_size=1)
    poisoned = inp.page_table.copy()
    cols = np.arange(poisoned.shape[1]) % 16 != 0
    poisoned[:, cols] = inp.num_slots + 1000 + np.arange(int(cols.sum()), dtype=np.int32)
    u.pt = up(poisoned)
    o16, l16 = u.decode(page_size=16)
    e16, el16 = u.extend(page_size=16)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o16), bits(o1))
    assert np.array_equal(l16.cpu().numpy().view(np.uint32), l1.cpu().numpy().view(np.uint32))
    assert np.array_equal(bits(e16), bits(e1))
    assert np.array_equal(el16.cpu().numpy().view(np.uint32), el1.cpu().numpy().view(np.uint32))
    kp, vp = oracle_pool(inp)
    ro, _ = oracle_decode(inp, kp, vp)
    assert_close(o16, ro, "decode page16 poisoned table")
    re, _ = oracle_extend(inp, kp, vp)
    assert_close(e16, re, "extend page16 poisoned table")


def test_extend_of_one_token_equals_decode():
    banner("extend(E=1) vs decode")
    inp = small_decode(91, 32, 8, [500, 1, 64, 1300], num_slots=4096)
    u = Uploaded(inp)
    u.store()
    od, ld = u.decode(split_tokens=4096)
    L = inp.dec_seq_lens
    oe, le = msgl.paged_extend(u.dq, u.k, u.v, u.pt, up((L - 1).astype(np.int32)),
                               up(np.ones_like(L)), up(np.arange(len(L) + 1, dtype=np.int32)),
                               1, int(L.max()), inp.sm_scale, req_rows=u.d_rows)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, _ = oracle_decode(inp, kp, vp)
    assert_close(oe, ro, "extend E=1")
    assert np.abs(f64(oe) - f64(od)).max() <= 2e-2


def test_extend_chunked_equals_full_prefill():
    banner("extend chunked vs full")
    N = 300
    inp = small_extend(92, 32, 8, [(0, N)], num_slots=2048)
    u = Uploaded(inp)
    u.store()
    full, _ = u.extend()
    row = inp.page_table[inp.ext_req_rows[0]][None, :]
    cuts = [0, 100, 229, N]
    kp, vp = oracle_pool(inp)
    ro, _ = oracle_extend(inp, kp, vp)
    for a, b in zip(cuts[:-1], cuts[1:]):
        oc, _ = msgl.paged_extend(u.eq[a:b].contiguous(), u.k, u.v, up(row.astype(np.int32)),
                                  up(np.array([a], np.int32)), up(np.array([b - a], np.int32)),
                                  up(np.array([0, b - a], np.int32)), b - a, b, inp.sm_scale)
        torch.cuda.synchronize()
        assert_close(oc, ro[a:b], f"chunk {a}:{b}")
        assert np.abs(f64(oc) - f64(full[a:b])).max() <= 2e-2


# ---------------------------------------------------------------------------
# sizes at the edges of the work split
# ---------------------------------------------------------------------------

def test_decode_one_request_cut_across_every_workgroup():
    """One request of 65,536 keys with the balanced split: its key line is
    cut into one range per workgroup, so the merge folds one partial per
    workgroup (eight at a time, many batches); also the fixed split at 512
    keys (128 chunks)."""
    banner("decode one 65,536-key request, balanced and fixed")
    inp = small_decode(140, 32, 8, [65536], num_slots=131072)
    u = Uploaded(inp)
    u.store()
    ob, lb = u.decode(split_tokens=0)
    of, lf = u.decode(split_tokens=512)
    torch.cuda.synchronize()
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(ob, ro, "decode 64K balanced")
    assert_lse_close(lb, rl, "decode 64K balanced lse")
    assert_close(of, ro, "decode 64K fixed 512")
    assert_lse_close(lf, rl, "decode 64K fixed 512 lse")


def test_decode_thousands_of_tiny_requests():
    """4,000 requests of 1-40 keys (a few empty): every workgroup's range
    holds dozens of request segments, most finished inside one workgroup,
    some cut at range ends."""
    banner("decode 4,000 tiny requests")
    rng = np.random.default_rng(141)
    lens = rng.integers(1, 41, 4000)
    inp = small_decode(141, 32, 8, lens, num_slots=262144)
    dl = inp.dec_seq_lens.copy()
    dl[[5, 1999, 3999]] = 0
    u = Uploaded(inp)
    u.store()
    out, lse = msgl.paged_decode(u.dq, u.k, u.v, u.pt, up(dl), u.d_max, inp.sm_scale,
                                 req_rows=u.d_rows, split_tokens=0)
    torch.cuda.synchronize()
    got = f64(out)
    assert np.all(got[[5, 1999, 3999]] == 0)
    assert np.all(np.isneginf(lse.cpu().numpy()[[5, 1999, 3999]]))
    sel = np.array(sorted(set(rng.choice(4000, 48, replace=False).tolist()) - {5, 1999, 3999}
                          | {0, 1, 2000, 3998}))
    kp, vp = oracle_pool(inp)
    ro, rl = oracle.paged_decode(inp.dec_q[sel], kp, vp, inp.page_table, inp.dec_req_rows[sel],
                                 dl[sel], inp.sm_scale, inp.num_kv_heads)
    t = torch.from_numpy(sel).cuda()
    assert_close(out[t], ro, "decode 4,000 tiny requests")
    assert_lse_close(lse[t], rl, "decode 4,000 tiny requests lse")


def test_extend_prefix_past_1024_key_tiles():
    """A 66,000-key prefix: its query tile visits 1,033 key tiles, more than
    the planner has length buckets, so the planner sorts by coarser buckets;
    planned and natural orders bitwise equal, sampled rows against the
    oracle (the long request and the short one)."""
    banner("extend with a 66,000-key prefix")
    inp = small_extend(142, 32, 8, [(66000, 70), (10, 300)], num_slots=131072)
    u = Uploaded(inp)
    u.store()
    op, lp = u.extend(plan=True)
    on, ln = u.extend(plan=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(op), bits(on))
    assert np.array_equal(lp.cpu().numpy().view(np.uint32), ln.cpu().numpy().view(np.uint32))
    rows = [0, 1, 33, 63, 64, 69, 70, 71, 200, 369]
    kp, vp = oracle_pool(inp)
    ro, rl = oracle.paged_extend(inp.ext_q, kp, vp, inp.page_table, inp.ext_req_rows,
                                 inp.ext_prefix_lens, inp.ext_extend_lens, inp.ext_q_offsets,
                                 inp.sm_scale, inp.num_kv_heads, query_subset=rows)
    t = torch.tensor(rows, device="cuda")
    assert_close(op[t], ro[rows], "extend 66K prefix")
    assert_lse_close(lp[t], rl[rows], "extend 66K prefix lse")


@pytest.mark.parametrize("P", [2, 8, 64, 256, 3])
def test_other_page_sizes_match_page_size_1(P):
    """Page sizes other than 16 on a table of P-slot pages (page permutation):
    decode (balanced and 96-key chunks) and extend bit-identical to
    page_size 1 on the same table, and held to the oracle.  For a power of
    two every non-first column of each page is overwritten by out-of-pool
    values first, so only page starts may be read; P = 3 (not a power of two)
    reads every column, so its table stays intact."""
    banner(f"page_size {P} vs 1")
    inp = small_extend(160 + P, 32, 8, [(3 * P + 5, 70), (0, 50)], page_size=P,
                       num_slots=max(16384, 64 * P), decode_lens=[700, 1, 2 * P + 1, 130])
    u = Uploaded(inp)
    u.store()
    d1, dl1 = u.decode(page_size=1)
    f1, fl1 = u.decode(page_size=1, split_tokens=96)
    e1, el1 = u.extend(page_size=1)
    if P & (P - 1) == 0:
        poisoned = inp.page_table.copy()
        cols = np.arange(poisoned.shape[1]) % P != 0
        poisoned[:, cols] = inp.num_slots + 7 + np.arange(int(cols.sum()), dtype=np.int32)
        u.pt = up(poisoned)
    dp, dlp = u.decode(page_size=P)
    fp, flp = u.decode(page_size=P, split_tokens=96)
    ep, elp = u.extend(page_size=P)
    torch.cuda.synchronize()
    for a, b, what in ((dp, d1, "decode"), (fp, f1, "decode 96-key chunks"), (ep, e1, "extend")):
        assert np.array_equal(bits(a), bits(b)), what
    for a, b, what in ((dlp, dl1, "decode lse"), (flp, fl1, "chunked lse"), (elp, el1, "extend lse")):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32)), what
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(dp, ro, f"decode page_size {P}")
    assert_lse_close(dlp, rl, f"decode page_size {P} lse")
    re, rel = oracle_extend(inp, kp, vp)
    assert_close(ep, re, f"extend page_size {P}")
    assert_lse_close(elp, rel, f"extend page_size {P} lse")


@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2), (8, 1)])
def test_tensor_parallel_shard_shapes_at_page_size_16(hq, hkv):
    """One tensor-parallel rank's share of the heads (one or two kv heads) on a
    table of 16-slot pages: balanced decode with requests cut across
    workgroups, the same decode with the new rows stored in the launch, and
    extend.  Every non-first column of each page is overwritten with
    out-of-pool values, so only page starts may be read.  Results are
    bit-identical to page_size 1 on the intact table and held to the oracle."""
    banner(f"shard hq={hq} hkv={hkv} page_size 16")
    P = 16
    inp = small_extend(190 + hq + hkv, hq, hkv, [(3 * P + 5, 70), (0, 50)], page_size=P,
                       num_slots=16384, decode_lens=[3000, 17, 900, 1, 2500])
    B = inp.num_decode
    u = Uploaded(inp)
    u.store()
    loc = up(inp.out_loc[-B:].astype(np.int32))

    def fused(ps):
        return msgl.store_kv_paged_decode(u.dq, u.k, u.v, u.k_new[-B:], u.v_new[-B:], loc, u.pt,
                                          u.d_lens, u.d_max, inp.sm_scale, req_rows=u.d_rows,
                                          page_size=ps)

    d1, dl1 = u.decode(page_size=1)
    f1, fl1 = fused(1)
    e1, el1 = u.extend(page_size=1)
    poisoned = inp.page_table.copy()
    cols = np.arange(poisoned.shape[1]) % P != 0
    poisoned[:, cols] = inp.num_slots + 7 + np.arange(int(cols.sum()), dtype=np.int32)
    u.pt = up(poisoned)
    dp, dlp = u.decode(page_size=P)
    fp, flp = fused(P)
    ep, elp = u.extend(page_size=P)
    torch.cuda.synchronize()
    for a, b, what in ((dp, d1, "decode"), (fp, f1, "fused store + decode"), (ep, e1, "extend")):
        assert np.array_equal(bits(a), bits(b)), what
    for a, b, what in ((dlp, dl1, "decode lse"), (flp, fl1, "fused lse"), (elp, el1, "extend lse")):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32)), what
    assert np.array_equal(bits(fp), bits(dp)), "fused vs two-call"
    kp, vp = oracle_pool(inp)
    ro, rl = oracle_decode(inp, kp, vp)
    assert_close(dp, ro, f"shard decode hq={hq} hkv={hkv}")
    assert_lse_close(dlp, rl, f"shard decode lse hq={hq} hkv={hkv}")
    re, rel = oracle_extend(inp, kp, vp)
    assert_close(ep, re, f"shard extend hq={hq} hkv={hkv}")
    assert_lse_close(elp, rel, f"shard extend lse hq={hq} hkv={hkv}")


def test_extend_q_from_a_merged_qkv_buffer_and_no_lse():
    """q as the attention layer hands it over after the prologue: the first
    Hq * 128 columns of a merged [T, (Hq + 2 Hkv) * 128] qkv buffer (row stride
    (Hq + 2 Hkv) * 128); the same call without an lse output.  Outputs equal
    the contiguous-q call bitwise."""
    banner("extend q strided in qkv, no lse")
    hq, hkv = 32, 8
    inp = small_extend(170, hq, hkv, [(40, 90), (0, 33)], num_slots=4096)
    u = Uploaded(inp)
    u.store()
    ref, ref_lse = u.extend()
    T = inp.ext_q.shape[0]
    qkv = torch.zeros((T, (hq + 2 * hkv) * 128), dtype=torch.bfloat16, device="cuda")
    qkv[:, :hq * 128] = u.eq.reshape(T, hq * 128)
    q = qkv[:, :hq * 128].view(T, hq, 128)
    assert q.stride(0) == (hq + 2 * hkv) * 128
    out, lse = msgl.paged_extend(q, u.k, u.v, u.pt, u.e_pre, u.e_ext, u.e_off, u.e_max, u.e_kv,
                                 inp.sm_scale, req_rows=u.e_rows)
    out2, lse2 = msgl.paged_extend(q, u.k, u.v, u.pt, u.e_pre, u.e_ext, u.e_off, u.e_max, u.e_kv,
                                   inp.sm_scale, req_rows=u.e_rows, want_lse=False)
    torch.cuda.synchronize()
    assert lse2 is None
    assert np.array_equal(bits(out), bits(ref)) and np.array_equal(bits(out2), bits(ref))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref_lse.cpu().numpy().view(np.uint32))
    kp, vp = oracle_pool(inp)
    ro, _ = oracle_extend(inp, kp, vp)
    assert_close(out, ro, "extend strided q")


@pytest.mark.parametrize("split", [0, 64])
def test_decode_without_lse_output(split):
    """No lse output (lse_out NULL): outputs equal the call that writes it,
    with requests finished in one workgroup and requests merged from parts."""
    banner(f"decode no lse split={split}")
    inp = small_decode(171, 32, 8, [3000, 5, 700, 64], num_slots=8192)
    u = Uploaded(inp)
    u.store()
    ref, _ = u.decode(split_tokens=split)
    out, lse = u.decode(split_tokens=split, want_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    assert np.array_equal(bits(out), bits(ref))


def test_extend_is_deterministic():
    """Three planned runs of a batch whose planner orders items with LDS
    atomics (so the dispatch order may differ run to run): bitwise equal."""
    banner("extend determinism")
    inp = small_extend(172, 32, 8, [(900, 300), (0, 257), (2048, 64), (100, 100), (5, 700)],
                       num_slots=8192)
    u = Uploaded(inp)
    u.store()
    outs = []
    for _ in range(3):
        o, l = u.extend()
        torch.cuda.synchronize()
        outs.append((bits(o), l.cpu().numpy().view(np.uint32)))
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
