"""GPU tests of the debug-check library (libmsgl_debug.so: the same sources
built with MSGL_DEBUG_CHECKS).

Good inputs give results bit-identical to the release library.  Each planted
bad index is one the checkers can see with every read in bounds (the table
row of a request is a real row, lengths stay within the table width or are
clamped to it before the table is scanned); the call must fail with
MSGL_ERR_INDEX, name the offending request, key or entry, and launch nothing
else: the pool keeps its bits.  Bad inputs go only through the debug library.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_attention_30_amd as msgl
from paged_kv_attention_30_amd import binding
from workloads import random_bf16, small_extend
from tests.gpu_util import Uploaded, up, bits

pytestmark = pytest.mark.gpu

INDEX = -7


def banner(msg):
    print(f"[gpu-debug-checks] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture
def dbg():
    with binding.using_library(binding.DEBUG_LIB_PATH) as lib:
        assert lib.msgl_debug_checks() == 1
        yield lib


def inputs(page_size=1):
    return small_extend(150, 32, 8, [(300, 90), (0, 70)], decode_lens=[700, 33, 129, 1],
                        page_size=page_size, num_slots=8192)


def expect_index_error(call, *words):
    with pytest.raises(msgl.MsglError) as e:
        call()
    assert e.value.status == INDEX, str(e.value)
    for w in words:
        assert w in str(e.value), str(e.value)
    return str(e.value)


def run_all(u, inp):
    """store, decode (balanced and fixed split), fused store + decode, extend."""
    u.store()
    od, ld = u.decode(split_tokens=0)
    of, lf = u.decode(split_tokens=64)
    ee, le = u.extend()
    B = inp.num_decode                               # the decode rows are the last B new rows
    loc = up(inp.out_loc[-B:].astype(np.int32))
    ofs, lfs = msgl.store_kv_paged_decode(u.dq, u.k, u.v, u.k_new[-B:], u.v_new[-B:], loc, u.pt,
                                          u.d_lens, u.d_max, inp.sm_scale, req_rows=u.d_rows)
    torch.cuda.synchronize()
    return [bits(u.k), bits(u.v), bits(od), ld.cpu().numpy(), bits(of), lf.cpu().numpy(),
            bits(ee), le.cpu().numpy(), bits(ofs), lfs.cpu().numpy()]


def test_good_calls_are_bit_identical_to_the_release_library(dbg):
    banner("debug build vs release on good inputs")
    inp = inputs()
    got = run_all(Uploaded(inp), inp)
    with binding.using_library(binding.LIB_PATH) as rel:
        assert rel.msgl_debug_checks() == 0
        ref = run_all(Uploaded(inp), inp)
    for i, (a, b) in enumerate(zip(got, ref)):
        assert np.array_equal(a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32),
                              b.view(np.uint16) if b.dtype == np.uint16 else b.view(np.uint32)), i


def test_store_with_an_out_of_pool_slot_is_refused(dbg):
    banner("store_kv: out_loc past the pool")
    inp = inputs()
    u = Uploaded(inp)
    before = (bits(u.k).copy(), bits(u.v).copy())
    loc = inp.out_loc.astype(np.int64).copy()
    loc[7] = inp.k_pool.shape[0]                     # one past the last slot
    expect_index_error(lambda: msgl.store_kv(u.k, u.v, u.k_new, u.v_new, up(loc)), "out_loc[7]")
    loc[7] = -3
    expect_index_error(lambda: msgl.store_kv(u.k, u.v, u.k_new, u.v_new, up(loc)), "out_loc[7]")
    torch.cuda.synchronize()
    assert np.array_equal(bits(u.k), before[0]) and np.array_equal(bits(u.v), before[1])
    # the report was cleared: a good call goes through
    msgl.store_kv(u.k, u.v, u.k_new, u.v_new, u.out_loc)
    torch.cuda.synchronize()


def test_decode_bad_table_entry_length_and_row_are_refused(dbg):
    banner("decode: table entry, seq_len and req_rows")
    inp = inputs()
    u = Uploaded(inp)
    u.store()
    pt = inp.page_table.copy()
    row = int(inp.dec_req_rows[1])
    pt[row, 5] = inp.k_pool.shape[0] + 3
    u.pt = up(pt)
    expect_index_error(lambda: u.decode(), "request 1", "key 5")
    u.pt = up(inp.page_table)
    lens = inp.dec_seq_lens.copy()
    lens[2] = u.d_max + 1                            # past the declared maximum
    expect_index_error(lambda: msgl.paged_decode(u.dq, u.k, u.v, u.pt, up(lens), u.d_max,
                                                 inp.sm_scale, req_rows=u.d_rows),
                       "request 2", "length")
    rows = inp.dec_req_rows.copy()
    rows[0] = -1
    expect_index_error(lambda: msgl.paged_decode(u.dq, u.k, u.v, u.pt, u.d_lens, u.d_max,
                                                 inp.sm_scale, req_rows=up(rows)),
                       "request 0", "req_rows")
    out, _ = u.decode()                               # good again
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_fused_store_must_write_the_newest_key(dbg):
    banner("fused store + decode: out_loc not the newest key's slot")
    inp = inputs()
    u = Uploaded(inp)
    u.store()
    before = (bits(u.k).copy(), bits(u.v).copy())
    B = inp.num_decode                               # the decode rows are the last B new rows
    loc = inp.out_loc[-B:].astype(np.int32).copy()
    row = int(inp.dec_req_rows[1])
    loc[1] = int(inp.page_table[row, 0])             # an older key of the same request
    expect_index_error(lambda: msgl.store_kv_paged_decode(
        u.dq, u.k, u.v, u.k_new[-B:], u.v_new[-B:], up(loc), u.pt, u.d_lens, u.d_max,
        inp.sm_scale, req_rows=u.d_rows), "request 1", "newest key")
    torch.cuda.synchronize()
    assert np.array_equal(bits(u.k), before[0]) and np.array_equal(bits(u.v), before[1])


def test_extend_bad_offsets_and_lengths_are_refused(dbg):
    banner("extend: q_offsets and extend_len")
    inp = inputs()
    u = Uploaded(inp)
    u.store()
    off = inp.ext_q_offsets.copy()
    off[1] += 1                                      # request 0's rows no longer span E
    expect_index_error(lambda: msgl.paged_extend(u.eq, u.k, u.v, u.pt, u.e_pre, u.e_ext, up(off),
                                                 u.e_max, u.e_kv, inp.sm_scale,
                                                 req_rows=u.e_rows), "request 0", "q_offsets")
    expect_index_error(lambda: msgl.paged_extend(u.eq, u.k, u.v, u.pt, u.e_pre, u.e_ext, u.e_off,
                                                 u.e_max - 1, u.e_kv, inp.sm_scale,
                                                 req_rows=u.e_rows), "length")
    out, _ = u.extend()
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()


def test_page_of_16_reaching_past_the_pool_is_refused(dbg):
    banner("page_size 16: a page start whose page runs past the pool")
    inp = inputs(page_size=16)
    u = Uploaded(inp)
    u.store()
    pt = inp.page_table.copy()
    row = int(inp.dec_req_rows[0])
    pt[row, 32] = inp.k_pool.shape[0] - 8            # keys 32..47 would read 8 slots past the end
    u.pt = up(pt)
    expect_index_error(lambda: u.decode(), "request 0", "key 32")


def test_prologue_with_an_out_of_pool_slot_is_refused(dbg):
    banner("prologue: out_loc past the pool")
    rng = np.random.default_rng(151)
    T, hq, hkv, S = 40, 32, 8, 1024
    qkv = up(random_bf16(rng, (T, (hq + 2 * hkv) * 128)))
    kp = up(random_bf16(rng, (S, hkv, 128)))
    vp = up(random_bf16(rng, (S, hkv, 128)))
    before = (bits(kp).copy(), bits(vp).copy())
    pos = up(np.arange(T, dtype=np.int32))
    cache = msgl.rope_cos_sin_cache(64, 128, 1e6)
    loc = np.arange(T, dtype=np.int32) * 3
    loc[11] = S
    expect_index_error(lambda: msgl.qk_norm_rope_store(qkv, kp, vp, pos, cache, up(loc), hq, hkv),
                       "out_loc[11]")
    torch.cuda.synchronize()
    assert np.array_equal(bits(kp), before[0]) and np.array_equal(bits(vp), before[1])


def test_full_mixed_batch_at_page_size_16_passes_the_checks(dbg):
    """The 127-request decode and the 6,144 + 2,048 extend at page_size 16
    (the mixed benchmark batch): every check passes and the results equal
    the release library's bit for bit."""
    from workloads import make_config
    banner("C5b through the debug-check library")
    inp = make_config("C5b")
    outs = []
    for path in (binding.DEBUG_LIB_PATH, binding.LIB_PATH):
        with binding.using_library(path):
            u = Uploaded(inp)
            u.store()
            od, ld = u.decode()
            oe, le = u.extend()
            torch.cuda.synchronize()
            outs.append((bits(od), ld.cpu().numpy().view(np.uint32), bits(oe),
                         le.cpu().numpy().view(np.uint32)))
            del u
            torch.cuda.empty_cache()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
