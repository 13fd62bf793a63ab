"""GPU tests of msgl_store_kv_paged_decode (store_kv of each request's new row
and the decode in one launch).

With out_loc[r] = page_table[row_r, seq_lens[r] - 1] a freshly allocated
slot, the one launch must leave the pool and the outputs bit-identical to
msgl_store_kv followed by msgl_paged_decode on the same inputs (the wave that
reads a request's newest key stores it first and reads it back once its own
store has completed).  Both paths run on separate copies of the same seeded
input; the fused results are also held to the oracle's tolerance.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_30_amd as msgl
from workloads import make_config, small_decode
from tests.gpu_util import Uploaded, up, bits, assert_close, assert_lse_close

pytestmark = pytest.mark.gpu


def banner(msg):
    print(f"[gpu-store-decode] {msg}", flush=True)
    sys.stdout.flush()


def separate(inp, lens, split, page_size, loc_dtype):
    u = Uploaded(inp)
    loc = up(inp.out_loc.astype(loc_dtype))
    msgl.store_kv(u.k, u.v, u.k_new, u.v_new, loc)
    out, lse = msgl.paged_decode(u.dq, u.k, u.v, u.pt, lens, u.d_max, inp.sm_scale,
                                 req_rows=u.d_rows, page_size=page_size, split_tokens=split)
    return u, out, lse


def fused(inp, lens, split, page_size, loc_dtype):
    u = Uploaded(inp)
    loc = up(inp.out_loc.astype(loc_dtype))
    out, lse = msgl.store_kv_paged_decode(u.dq, u.k, u.v, u.k_new, u.v_new, loc, u.pt, lens,
                                          u.d_max, inp.sm_scale, req_rows=u.d_rows,
                                          page_size=page_size, split_tokens=split)
    return u, out, lse


def assert_same(a, b, what):
    ua, oa, la = a
    ub, ob, lb = b
    torch.cuda.synchronize()
    assert torch.equal(ua.k.view(torch.int16), ub.k.view(torch.int16)), f"{what}: K pools differ"
    assert torch.equal(ua.v.view(torch.int16), ub.v.view(torch.int16)), f"{what}: V pools differ"
    assert np.array_equal(bits(oa), bits(ob)), f"{what}: outputs differ"
    assert np.array_equal(la.cpu().numpy().view(np.uint32), lb.cpu().numpy().view(np.uint32)), \
        f"{what}: lse differ"


CASES = [
    # (hq, hkv, seq_lens, split_tokens, page_size, out_loc dtype)
    (32, 8, [700, 1, 129, 1024, 513, 2], 0, 1, np.int32),
    (32, 8, [700, 1, 129, 1024, 513, 2], 0, 1, np.int64),
    (32, 8, [700, 1, 129, 1024, 513], 64, 1, np.int64),
    (16, 8, [1, 31, 32, 33, 64, 65], 0, 1, np.int32),
    (64, 8, [1500, 2048, 3, 777], 256, 1, np.int32),
    (16, 1, [300, 45], 0, 1, np.int32),
    (32, 2, [90, 1000, 1001], 128, 1, np.int64),
    (32, 8, [160, 33, 1000, 17], 0, 16, np.int32),
    # GQA ratio 8 in balanced mode (the long-tail batch's launch), lengths
    # past 4K keys so requests are cut across workgroups
    (64, 8, [5000, 1024, 7, 2048, 4711, 1300, 64, 3333], 0, 1, np.int64),
    # kv heads spread over two and four workgroups: each stores its own heads'
    # slices of the new rows
    (16, 16, [700, 1, 129, 2000, 33], 0, 1, np.int32),
    (32, 32, [300, 1025, 64], 0, 1, np.int64),
    (16, 16, [700, 1, 129, 2000, 33], 128, 1, np.int32),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_equals_store_then_decode(case):
    hq, hkv, lens, split, ps, ldt = CASES[case]
    banner(f"hq={hq} hkv={hkv} lens={lens} split={split} page_size={ps} out_loc={ldt.__name__}")
    inp = small_decode(90 + case, hq, hkv, lens, page_size=ps,
                       num_slots=max(8192, -(-2 * sum(lens) // 4096) * 4096))
    d_lens = up(inp.dec_seq_lens)
    a = separate(inp, d_lens, split, ps, ldt)
    b = fused(inp, d_lens, split, ps, ldt)
    assert_same(a, b, f"case {case}")
    kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    ro, rl = oracle.paged_decode(inp.dec_q, kp, vp, inp.page_table, inp.dec_req_rows,
                                 inp.dec_seq_lens, inp.sm_scale, inp.num_kv_heads)
    assert_close(b[1], ro, f"fused case {case}")
    assert_lse_close(b[2], rl, f"fused case {case}")


@pytest.mark.parametrize("lens_kind", ["many", "tiny", "straddle", "empty"])
def test_fused_more_rows_than_workgroups_and_empty_requests(lens_kind):
    """300 requests (more new rows than resident workgroups: a workgroup
    stores several); 1-4 keys each (the newest key is often a segment's only
    key); lengths of 33-95 keys (the newest key in the first or the second
    wave's tile); or empty requests (their row is still stored)."""
    banner(f"fused {lens_kind}")
    rng = np.random.default_rng(11)
    if lens_kind == "many":
        lens = rng.integers(1, 400, 300)
    elif lens_kind == "tiny":
        lens = rng.integers(1, 5, 300)
    elif lens_kind == "straddle":
        lens = rng.integers(33, 96, 200)
    else:
        lens = rng.integers(1, 900, 40)
    inp = small_decode(98, 32, 8, lens, num_slots=1 << 18)
    dl = inp.dec_seq_lens.copy()
    if lens_kind == "empty":
        dl[[0, 17, 39]] = 0
    d_lens = up(dl)
    a = separate(inp, d_lens, 0, 1, np.int32)
    b = fused(inp, d_lens, 0, 1, np.int32)
    assert_same(a, b, lens_kind)
    if lens_kind == "empty":
        out = b[1].float().cpu().numpy()
        assert np.all(out[[0, 17, 39]] == 0)
        assert np.all(np.isneginf(b[2].cpu().numpy()[[0, 17, 39]]))
    # a spread of requests against the oracle, at the lengths the GPU saw
    # (the emptied requests are checked above)
    n = len(lens)
    picked = {0, 1, 2, n // 3, n // 2, n - 2, n - 1, int(np.argmax(lens))}
    sel = np.array(sorted(picked - ({0, 17, 39} if lens_kind == "empty" else set())))
    kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    ro, rl = oracle.paged_decode(inp.dec_q[sel], kp, vp, inp.page_table, inp.dec_req_rows[sel],
                                 dl[sel], inp.sm_scale, inp.num_kv_heads)
    t = torch.from_numpy(sel).cuda()
    assert_close(b[1][t], ro, f"fused {lens_kind}")
    assert_lse_close(b[2][t], rl, f"fused {lens_kind}")


def test_fused_one_chunk_per_request_and_identity_rows():
    """Fixed chunks wider than every request (one chunk each, no workspace)
    and no req_rows (request r reads table row r)."""
    banner("fused one chunk, identity rows")
    inp = small_decode(120, 32, 8, [700, 1, 129, 33], num_slots=4096)
    # the identity mapping needs the table rows in request order
    inp.page_table = np.ascontiguousarray(inp.page_table[inp.dec_req_rows])
    inp.dec_req_rows = np.arange(inp.num_decode, dtype=np.int32)
    d_lens = up(inp.dec_seq_lens)
    runs = []
    for fused_call in (False, True):
        u = Uploaded(inp)
        loc = up(inp.out_loc.astype(np.int32))
        if fused_call:
            out, lse = msgl.store_kv_paged_decode(u.dq, u.k, u.v, u.k_new, u.v_new, loc, u.pt,
                                                  d_lens, u.d_max, inp.sm_scale,
                                                  split_tokens=1024)
        else:
            msgl.store_kv(u.k, u.v, u.k_new, u.v_new, loc)
            out, lse = msgl.paged_decode(u.dq, u.k, u.v, u.pt, d_lens, u.d_max, inp.sm_scale,
                                         split_tokens=1024)
        runs.append((u, out, lse))
    assert_same(runs[0], runs[1], "one chunk")
    kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    ro, rl = oracle.paged_decode(inp.dec_q, kp, vp, inp.page_table, inp.dec_req_rows,
                                 inp.dec_seq_lens, inp.sm_scale, inp.num_kv_heads)
    assert_close(runs[1][1], ro, "fused one chunk")
    assert_lse_close(runs[1][2], rl, "fused one chunk")


def test_fused_full_c2_in_the_bench_launch():
    """The 64-request, 512K-slot decode batch as the benchmark times it."""
    banner("fused C2 full size")
    inp = make_config("C2")
    d_lens = up(inp.dec_seq_lens)
    a = separate(inp, d_lens, 0, 1, np.int64)
    del a[0].k_new, a[0].v_new
    b = fused(inp, d_lens, 0, 1, np.int64)
    assert_same(a, b, "C2")
    del a
    torch.cuda.empty_cache()
    L = inp.dec_seq_lens
    sel = np.array(sorted({int(np.argmax(L)), int(np.argmin(L)), 0, len(L) - 1, 20, 41}))
    kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    ro, rl = oracle.paged_decode(inp.dec_q[sel], kp, vp, inp.page_table, inp.dec_req_rows[sel],
                                 L[sel], inp.sm_scale, inp.num_kv_heads)
    t = torch.from_numpy(sel).cuda()
    assert_close(b[1][t], ro, "fused C2")
    assert_lse_close(b[2][t], rl, "fused C2")


def test_fused_full_c4_in_the_bench_launch():
    """The 256-request long-tail batch (Hq 64 / Hkv 8, kv lengths up to 23K)
    through the one store + decode launch the benchmark times: balanced split,
    requests cut across workgroups and merged."""
    banner("fused C4 full size")
    inp = make_config("C4")
    d_lens = up(inp.dec_seq_lens)
    a = separate(inp, d_lens, 0, 1, np.int64)
    del a[0].k_new, a[0].v_new, a[0].dq
    b = fused(inp, d_lens, 0, 1, np.int64)
    assert_same(a, b, "C4")
    del a
    torch.cuda.empty_cache()
    L = inp.dec_seq_lens
    sel = np.array(sorted({int(np.argmax(L)), int(np.argmin(L)), 0, len(L) - 1, 37, 128, 201}))
    kp, vp = oracle.store_kv(inp.k_pool, inp.v_pool, inp.k_new, inp.v_new, inp.out_loc)
    ro, rl = oracle.paged_decode(inp.dec_q[sel], kp, vp, inp.page_table, inp.dec_req_rows[sel],
                                 L[sel], inp.sm_scale, inp.num_kv_heads)
    t = torch.from_numpy(sel).cuda()
    assert_close(b[1][t], ro, "fused C4")
    assert_lse_close(b[2][t], rl, "fused C4")
