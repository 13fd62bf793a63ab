"""The C ABI: symbols, status strings and host-side validation (CPU only).

Validation runs before any HIP call, so every rejected call below returns
its status code on a machine without a GPU.  Pointers passed here are fake
(never dereferenced); calls that would pass validation are not made.
"""

import ctypes
import os
import re

import pytest

import paged_kv_attention_30_amd as msgl
from paged_kv_attention_30_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msgl.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH, INDEX = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 0x10000          # 64 KiB-aligned fake device address, never touched
FAKE2 = 0x20000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(msgl_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return msgl.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), f"{name} declared in msgl.h but not exported"
        assert name in binding.SIGNATURES, f"{name} has no ctypes signature"


def test_every_kvcache_symbol_is_exported(lib):
    from paged_kv_attention_30_amd import kvcache
    text = open(os.path.join(ROOT, "include", "msgl_kvcache.h")).read()
    names = sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(msgl_\w+)\s*\(", text, re.M)))
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), f"{name} declared in msgl_kvcache.h but not exported"
        assert name in kvcache._SIGS, f"{name} has no ctypes signature"


def test_status_strings_and_version(lib):
    assert lib.msgl_version() >= 100
    for code in (OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH, INDEX):
        assert lib.msgl_status_string(code)
    assert b"debug-check" in lib.msgl_status_string(INDEX)
    assert b"unknown" in lib.msgl_status_string(-99)


def test_release_and_debug_check_builds():
    """The release library trusts device indices; the debug-check build of the
    same sources reports itself and validates host arguments the same way."""
    import ctypes as ct
    rel = msgl.load()
    assert rel.msgl_debug_checks() == 0
    dbg = ct.CDLL(binding.DEBUG_LIB_PATH)
    dbg.msgl_debug_checks.restype = ct.c_int
    assert dbg.msgl_debug_checks() == 1
    with binding.using_library(binding.DEBUG_LIB_PATH) as lib:
        assert lib.msgl_debug_checks() == 1
        assert extend(lib, causal=0) == UNSUP
        assert decode(lib, k=None) == NULL
    assert msgl.load().msgl_debug_checks() == 0


def decode(lib, **kw):
    args = dict(out=FAKE, lse=FAKE, q=FAKE, q_stride=32 * 128, k=FAKE, v=FAKE2, slots=1024,
                cstride=8 * 128, pt=FAKE, pt_stride=4096, rows=None, lens=FAKE, batch=4, hq=32,
                hkv=8, d=128, page=1, max_len=4096, scale=0.088, split=0, ws=None, ws_bytes=0)
    args.update(kw)
    return lib.msgl_paged_decode(args["out"], args["lse"], args["q"], args["q_stride"], args["k"],
                                 args["v"], args["slots"], args["cstride"], args["pt"],
                                 args["pt_stride"], args["rows"], args["lens"], args["batch"],
                                 args["hq"], args["hkv"], args["d"], args["page"], args["max_len"],
                                 args["scale"], args["split"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), NULL),
    (dict(out=None), NULL),
    (dict(lens=None), NULL),
    (dict(d=64), UNSUP),
    (dict(hq=24), UNSUP),            # ratio 3
    (dict(hq=7), UNSUP),             # not a multiple of hkv
    (dict(hkv=0), SHAPE),
    (dict(batch=-1), SHAPE),
    (dict(cstride=100), SHAPE),
    (dict(q_stride=1000), SHAPE),
    (dict(pt_stride=100), SHAPE),
    (dict(split=48), SHAPE),
    (dict(page=0), UNSUP),
    (dict(k=FAKE + 2), ALIGN),
    (dict(q=FAKE + 4), ALIGN),
    (dict(cstride=8 * 128 + 4), ALIGN),
    (dict(ws=None, ws_bytes=0), WS),           # 4096 keys need more than one chunk
    (dict(ws=FAKE + 64, ws_bytes=1 << 30), WS),  # misaligned workspace
])
def test_decode_validation(lib, kw, code):
    st = decode(lib, **kw)
    assert st == code, (st, lib.msgl_last_error())
    assert lib.msgl_last_error()  # a message with a source location
    assert b"api.hip" in lib.msgl_last_error()


def test_decode_empty_batch_is_a_no_op(lib):
    assert decode(lib, batch=0) == OK


def fused(lib, **kw):
    args = dict(out=FAKE, lse=FAKE, q=FAKE, q_stride=32 * 128, k=FAKE, v=FAKE2, slots=1024,
                cstride=8 * 128, knew=FAKE, vnew=FAKE2, nstride=8 * 128, loc=FAKE, idx=0,
                pt=FAKE, pt_stride=4096, rows=None, lens=FAKE, batch=4, hq=32, hkv=8, d=128,
                page=1, max_len=4096, scale=0.088, split=0, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    a = args
    return lib.msgl_store_kv_paged_decode(
        a["out"], a["lse"], a["q"], a["q_stride"], a["k"], a["v"], a["slots"], a["cstride"],
        a["knew"], a["vnew"], a["nstride"], a["loc"], a["idx"], a["pt"], a["pt_stride"],
        a["rows"], a["lens"], a["batch"], a["hq"], a["hkv"], a["d"], a["page"], a["max_len"],
        a["scale"], a["split"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(knew=None), NULL),
    (dict(vnew=None), NULL),
    (dict(loc=None), NULL),
    (dict(knew=FAKE + 8), ALIGN),
    (dict(nstride=8 * 128 + 4), ALIGN),
    (dict(nstride=100), SHAPE),
    (dict(idx=7), UNSUP),
    (dict(loc=FAKE + 2), ALIGN),
    (dict(idx=1, loc=FAKE + 4), ALIGN),
    (dict(k=None), NULL),            # the decode's own checks come first
    (dict(hq=24), UNSUP),
    (dict(ws=None, ws_bytes=0), WS),
])
def test_store_decode_validation(lib, kw, code):
    st = fused(lib, **kw)
    assert st == code, (st, lib.msgl_last_error())
    assert b"api.hip" in lib.msgl_last_error()


def test_store_decode_empty_batch_is_a_no_op(lib):
    assert fused(lib, batch=0) == OK


def test_decode_workspace_size_rule(lib):
    # balanced ranges (split 0): partials for up to 2048 workgroups + batch
    n, s = msgl.paged_decode_workspace_size(64, 32, 8, 4096, 0)
    assert s == 0
    assert n >= (2048 + 64) * 32 * (128 + 1) * 4 + 64 * 2 * 4
    assert msgl.paged_decode_workspace_size(5, 32, 8, 10, 0)[0] > 0
    # fixed chunks: one partial per (chunk, request); none when one chunk suffices
    n, s = msgl.paged_decode_workspace_size(64, 32, 8, 4096, 256)
    assert s == 256 and n >= 16 * 64 * 32 * 129 * 4
    assert msgl.paged_decode_workspace_size(64, 32, 8, 200, 256)[0] == 0
    assert msgl.paged_decode_workspace_size(0, 32, 8, 200, 256)[0] == 0


def extend(lib, **kw):
    args = dict(out=FAKE, lse=FAKE, q=FAKE, q_stride=32 * 128, k=FAKE, v=FAKE2, slots=1024,
                cstride=8 * 128, pt=FAKE, pt_stride=4096, rows=None, pre=FAKE, ext=FAKE, off=FAKE,
                batch=2, hq=32, hkv=8, d=128, page=1, max_ext=512, max_kv=4096, scale=0.088,
                causal=1, ws=None, ws_bytes=0)
    args.update(kw)
    return lib.msgl_paged_extend(args["out"], args["lse"], args["q"], args["q_stride"], args["k"],
                                 args["v"], args["slots"], args["cstride"], args["pt"],
                                 args["pt_stride"], args["rows"], args["pre"], args["ext"],
                                 args["off"], args["batch"], args["hq"], args["hkv"], args["d"],
                                 args["page"], args["max_ext"], args["max_kv"], args["scale"],
                                 args["causal"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(causal=0), UNSUP),
    (dict(pre=None), NULL),
    (dict(off=None), NULL),
    (dict(max_kv=100), SHAPE),
    (dict(pt_stride=1000), SHAPE),
    (dict(d=256), UNSUP),
    (dict(hq=40), UNSUP),
    (dict(out=FAKE + 8), ALIGN),
    (dict(batch=-2), SHAPE),
])
def test_extend_validation(lib, kw, code):
    st = extend(lib, **kw)
    assert st == code, (st, lib.msgl_last_error())


def test_extend_workspace_rule(lib):
    # 256 query rows per workgroup: ratio 4 -> 64 positions per query tile
    assert msgl.paged_extend_workspace_size(8, 32, 8, 2048, 10240) == 16 + 4 * 8 * 32
    assert msgl.paged_extend_workspace_size(3, 16, 16, 300, 300) == 16 + 4 * 3 * 2
    assert msgl.paged_extend_workspace_size(1, 64, 4, 17, 17) == 16 + 4 * 1 * 2
    assert msgl.paged_extend_workspace_size(0, 32, 8, 2048, 2048) == 0
    assert msgl.paged_extend_workspace_size(4, 32, 8, 0, 2048) == 0
    # batch 2, max_ext 512 -> 8 query tiles each
    need = 16 + 4 * 2 * 8
    assert extend(lib, ws=FAKE, ws_bytes=need - 4) == WS
    assert extend(lib, ws=FAKE + 8, ws_bytes=need) == ALIGN


def test_extend_zero_length_is_a_no_op(lib):
    assert extend(lib, max_ext=0) == OK
    assert extend(lib, batch=0) == OK


def test_store_validation(lib):
    def store(**kw):
        a = dict(k=FAKE, v=FAKE2, slots=1024, cstride=1024, kn=FAKE, vn=FAKE2, nstride=1024,
                 loc=FAKE, idx=0, n=4, hkv=8, d=128, dtype=0)
        a.update(kw)
        return lib.msgl_store_kv(a["k"], a["v"], a["slots"], a["cstride"], a["kn"], a["vn"],
                                 a["nstride"], a["loc"], a["idx"], a["n"], a["hkv"], a["d"],
                                 a["dtype"], None)
    assert store(n=0) == OK
    assert store(n=-1) == SHAPE
    assert store(loc=None) == NULL
    assert store(dtype=7) == UNSUP
    assert store(idx=3) == UNSUP
    assert store(cstride=512) == SHAPE
    assert store(nstride=512) == SHAPE
    assert store(k=FAKE + 1) == ALIGN
    assert store(loc=FAKE + 2) == ALIGN
    assert store(idx=1, loc=FAKE + 4) == ALIGN


def test_merge_validation(lib):
    def merge(**kw):
        a = dict(out=FAKE, lse=FAKE, po=FAKE, pl=FAKE2, parts=3, n=5, h=8, d=128, dt=0)
        a.update(kw)
        return lib.msgl_merge_states(a["out"], a["lse"], a["po"], a["pl"], a["parts"], a["n"],
                                     a["h"], a["d"], a["dt"], None)
    assert merge(n=0) == OK
    assert merge(parts=0) == SHAPE
    assert merge(d=130) == UNSUP
    assert merge(d=512) == UNSUP
    assert merge(dt=5) == UNSUP
    assert merge(po=None) == NULL
    assert merge(po=FAKE + 4) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(2, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        msgl.paged_decode(q, q, q, torch.zeros(2, 4, dtype=torch.int32),
                          torch.ones(2, dtype=torch.int32), 4, 0.1)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.load(str(tmp_path / "nope.so"))
    monkeypatch.setattr(binding, "_lib", None)
    binding.load()


def test_embedding_gather_validation(lib):
    def gather(**kw):
        a = dict(out=FAKE, ostride=64, w=FAKE2, rows=100, wstride=64, ids=FAKE, idx=0, n=8,
                 start=0, hidden=64, dtype=0)
        a.update(kw)
        return lib.msgl_embedding_gather(a["out"], a["ostride"], a["w"], a["rows"], a["wstride"],
                                         a["ids"], a["idx"], a["n"], a["start"], a["hidden"],
                                         a["dtype"], None)
    assert gather(n=0) == OK
    assert gather(n=-1) == SHAPE
    assert gather(rows=-1) == SHAPE
    assert gather(hidden=0) == SHAPE
    assert gather(ostride=32) == SHAPE
    assert gather(wstride=10) == SHAPE
    assert gather(dtype=3) == UNSUP
    assert gather(idx=2) == UNSUP
    assert gather(ids=None) == NULL
    assert gather(w=None) == NULL
    assert gather(out=FAKE + 1) == ALIGN
    assert gather(idx=1, ids=FAKE + 4) == ALIGN


def test_decode_graph_layout_rule(lib):
    """The graph runner's buffer layout (host-only): regions in the documented
    order, 256-byte aligned, each large enough, the decode workspace last."""
    import ctypes
    off = (ctypes.c_size_t * 10)()
    assert lib.msgl_decode_graph_layout(64, 32, 8, 128, 4096, off) == OK
    o = list(off)
    need = [64 * 32 * 128 * 2, 64 * 8 * 128 * 2, 64 * 8 * 128 * 2, 64 * 32 * 128 * 2, 64 * 32 * 4,
            64 * 4, 64 * 4, 64 * 4,
            binding.paged_decode_workspace_size(64, 32, 8, 4096)[0]]
    for i in range(9):
        assert o[i] % 256 == 0
        assert o[i + 1] - o[i] >= need[i]
    assert lib.msgl_decode_graph_layout(0, 32, 8, 128, 4096, off) == SHAPE
    assert lib.msgl_decode_graph_layout(4, 32, 8, 64, 4096, off) == SHAPE
    assert lib.msgl_decode_graph_layout(4, 32, 8, 128, 4096, None) == SHAPE
    h = ctypes.c_void_p()
    assert lib.msgl_decode_graph_create(None, None, 0, 0, None, 0, 32, 8, 128, 1, 4, 64, 0.1, 0, 0,
                                        0, None, 0, ctypes.byref(h)) == NULL
    assert lib.msgl_decode_graph_run(None, 1, None) == NULL
    assert lib.msgl_decode_graph_bucket(None, 1) == -1


def test_prologue_validation(lib):
    def pro(**kw):
        a = dict(q=FAKE, qs=32 * 128, k=FAKE, v=FAKE2, slots=1024, cs=8 * 128, qkv=FAKE,
                 qkvs=48 * 128, qw=None, kw=None, eps=1e-6, pos=FAKE, cache=FAKE, maxpos=4096,
                 loc=FAKE, idx=0, n=4, hq=32, hkv=8, d=128)
        a.update(kw)
        return lib.msgl_qk_norm_rope_store(a["q"], a["qs"], a["k"], a["v"], a["slots"], a["cs"],
                                           a["qkv"], a["qkvs"], a["qw"], a["kw"], a["eps"], a["pos"],
                                           a["cache"], a["maxpos"], a["loc"], a["idx"], a["n"],
                                           a["hq"], a["hkv"], a["d"], None)
    assert pro(n=0) == OK
    assert pro(n=-1) == SHAPE
    assert pro(idx=7) == UNSUP
    assert pro(d=64) == UNSUP
    assert pro(hq=24) == UNSUP
    assert pro(qkvs=40 * 128) == SHAPE
    assert pro(qs=16 * 128) == SHAPE
    assert pro(maxpos=0) == SHAPE
    assert pro(eps=-1.0) == SHAPE
    assert pro(pos=None) == NULL
    assert pro(q=FAKE + 8) == ALIGN
    assert pro(qkvs=48 * 128 + 4) == ALIGN
    assert pro(cs=8 * 128 + 4) == ALIGN          # pool rows must stay 16-byte aligned
    assert pro(k=FAKE + 8) == ALIGN


# ---------------------------------------------------------------------------
# msgl_validate_*: the same checks with no HIP call, so valid arguments can be
# checked on a host without a GPU (every call below would otherwise launch)
# ---------------------------------------------------------------------------

def _validate_decode(lib, fused_call=False, **kw):
    a = dict(out=FAKE, lse=FAKE, q=FAKE, q_stride=32 * 128, k=FAKE, v=FAKE2, slots=1024,
             cstride=8 * 128, knew=FAKE, vnew=FAKE2, nstride=8 * 128, loc=FAKE, idx=0,
             pt=FAKE, pt_stride=4096, rows=None, lens=FAKE, batch=4, hq=32, hkv=8, d=128,
             page=1, max_len=4096, scale=0.088, split=0, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    if fused_call:
        return lib.msgl_validate_store_kv_paged_decode(
            a["out"], a["lse"], a["q"], a["q_stride"], a["k"], a["v"], a["slots"], a["cstride"],
            a["knew"], a["vnew"], a["nstride"], a["loc"], a["idx"], a["pt"], a["pt_stride"],
            a["rows"], a["lens"], a["batch"], a["hq"], a["hkv"], a["d"], a["page"],
            a["max_len"], a["scale"], a["split"], a["ws"], a["ws_bytes"])
    return lib.msgl_validate_paged_decode(
        a["out"], a["lse"], a["q"], a["q_stride"], a["k"], a["v"], a["slots"], a["cstride"],
        a["pt"], a["pt_stride"], a["rows"], a["lens"], a["batch"], a["hq"], a["hkv"], a["d"],
        a["page"], a["max_len"], a["scale"], a["split"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("fused_call", [False, True])
def test_validate_decode_accepts_valid_arguments(lib, fused_call):
    assert _validate_decode(lib, fused_call) == OK, lib.msgl_last_error()
    assert lib.msgl_last_error() == b""
    # fixed chunks, a GQA ratio of 8, page_size 16, identity rows left out, no lse
    assert _validate_decode(lib, fused_call, split=256, hq=64, q_stride=64 * 128, page=16,
                            lse=None) == OK
    # fixed chunks with one chunk per request need no workspace
    assert _validate_decode(lib, fused_call, split=4096, ws=None, ws_bytes=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), NULL), (dict(d=64), UNSUP), (dict(cstride=100), SHAPE),
    (dict(q=FAKE + 4), ALIGN), (dict(ws=None, ws_bytes=0), WS), (dict(split=48), SHAPE),
])
def test_validate_decode_returns_the_call_status(lib, kw, code):
    assert _validate_decode(lib, **kw) == code
    assert decode(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(knew=None), NULL), (dict(idx=7), UNSUP), (dict(nstride=100), SHAPE),
    (dict(knew=FAKE + 8), ALIGN),
])
def test_validate_store_decode_returns_the_call_status(lib, kw, code):
    assert _validate_decode(lib, True, **kw) == code
    assert fused(lib, **kw) == code


def test_validate_store_kv(lib):
    def v(**kw):
        a = dict(k=FAKE, v=FAKE2, slots=1024, cstride=8 * 128, knew=FAKE, vnew=FAKE2,
                 nstride=8 * 128, loc=FAKE, idx=1, n=64, hkv=8, d=128, dtype=0)
        a.update(kw)
        return lib.msgl_validate_store_kv(a["k"], a["v"], a["slots"], a["cstride"], a["knew"],
                                          a["vnew"], a["nstride"], a["loc"], a["idx"], a["n"],
                                          a["hkv"], a["d"], a["dtype"])
    assert v() == OK and v(dtype=1, idx=0) == OK and v(n=0, loc=None) == OK
    assert v(loc=None) == NULL and v(idx=3) == UNSUP and v(nstride=100) == SHAPE
    assert v(n=-1) == SHAPE and v(dtype=5) == UNSUP


def test_validate_extend(lib):
    def v(**kw):
        a = dict(out=FAKE, lse=FAKE, q=FAKE, q_stride=32 * 128, k=FAKE, v=FAKE2, slots=1024,
                 cstride=8 * 128, pt=FAKE, pt_stride=4096, rows=None, pre=FAKE, ext=FAKE,
                 off=FAKE, batch=2, hq=32, hkv=8, d=128, page=1, max_ext=512, max_kv=4096,
                 scale=0.088, causal=1, ws=FAKE, ws_bytes=1 << 20)
        a.update(kw)
        return lib.msgl_validate_paged_extend(
            a["out"], a["lse"], a["q"], a["q_stride"], a["k"], a["v"], a["slots"], a["cstride"],
            a["pt"], a["pt_stride"], a["rows"], a["pre"], a["ext"], a["off"], a["batch"],
            a["hq"], a["hkv"], a["d"], a["page"], a["max_ext"], a["max_kv"], a["scale"],
            a["causal"], a["ws"], a["ws_bytes"])
    assert v() == OK and v(ws=None, ws_bytes=0) == OK and v(hq=8, page=16) == OK
    assert v(causal=0) == UNSUP and v(pre=None) == NULL and v(ws_bytes=8) == WS
    assert v(max_kv=100) == SHAPE


def test_validate_merge_states(lib):
    def v(**kw):
        a = dict(out=FAKE, lse=FAKE, po=FAKE, pl=FAKE2, parts=4, n=64, heads=32, d=128, dt=0)
        a.update(kw)
        return lib.msgl_validate_merge_states(a["out"], a["lse"], a["po"], a["pl"], a["parts"],
                                              a["n"], a["heads"], a["d"], a["dt"])
    assert v() == OK and v(dt=1, lse=None) == OK and v(n=0, out=None) == OK
    assert v(parts=0) == SHAPE and v(po=None) == NULL and v(d=6) == UNSUP
    assert v(po=FAKE + 4) == ALIGN
