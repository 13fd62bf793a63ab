"""Thin Python binding over the libmsgl C ABI (argument marshalling only).

Every function takes torch tensors that already live on the GPU, checks
dtypes/devices/contiguity, passes raw pointers and sizes to the library and
enqueues the work on torch's current HIP stream (or the ``stream`` given).
All computation happens in the HIP kernels; nothing here computes results.
If the library is missing, loading fails loudly: there is no fallback.
"""

from __future__ import annotations

import contextlib
import ctypes
import os

import torch

from ._build import DEBUG_LIB_PATH, LIB_PATH

MSGL_OK = 0
DTYPE_BF16 = 0
DTYPE_F32 = 1
INDEX_I32 = 0
INDEX_I64 = 1

_lib = None

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_size_t = ctypes.c_size_t

SIGNATURES = {
    "msgl_version": (_i32, []),
    "msgl_debug_checks": (_i32, []),
    "msgl_status_string": (ctypes.c_char_p, [_i32]),
    "msgl_last_error": (ctypes.c_char_p, []),
    "msgl_store_kv": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i64,
                             _c_void_p, _i32, _i64, _i32, _i32, _i32, _c_void_p]),
    "msgl_paged_decode": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _c_void_p,
                                 _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _f32, _i32, _c_void_p, _size_t,
                                 _c_void_p]),
    "msgl_store_kv_paged_decode": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                                          _c_void_p, _i64, _i64, _c_void_p, _c_void_p, _i64,
                                          _c_void_p, _i32, _c_void_p, _i64, _c_void_p,
                                          _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                          _i32, _c_void_p, _size_t, _c_void_p]),
    "msgl_store_kv_paged_decode_noalloc": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64,
                                                  _c_void_p, _c_void_p, _i64, _i64, _c_void_p,
                                                  _c_void_p, _i64, _c_void_p, _i32, _c_void_p,
                                                  _i64, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                                  _i32, _i32, _i32, _f32, _i32, _c_void_p]),
    "msgl_paged_decode_workspace_size": (_size_t, [_i32, _i32, _i32, _i32, _i32, _i32,
                                                   ctypes.POINTER(_i32)]),
    "msgl_paged_extend": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _c_void_p,
                                 _i64, _i64, _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p,
                                 _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                 _i32, _c_void_p, _size_t, _c_void_p]),
    "msgl_paged_extend_workspace_size": (_size_t, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "msgl_merge_states": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32,
                                 _i32, _i32, _c_void_p]),
    "msgl_embedding_gather": (_i32, [_c_void_p, _i64, _c_void_p, _i64, _i64, _c_void_p, _i32,
                                     _i64, _i64, _i32, _i32, _c_void_p]),
    "msgl_rope_cos_sin_cache": (_i32, [_c_void_p, _i64, _i32, ctypes.c_double, _c_void_p]),
    "msgl_qk_norm_rope_store": (_i32, [_c_void_p, _i64, _c_void_p, _c_void_p, _i64, _i64,
                                       _c_void_p, _i64, _c_void_p, _c_void_p, _f32, _c_void_p,
                                       _c_void_p, _i64, _c_void_p, _i32, _i64, _i32, _i32, _i32,
                                       _c_void_p]),
    "msgl_validate_store_kv": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _c_void_p,
                                      _i64, _c_void_p, _i32, _i64, _i32, _i32, _i32]),
    "msgl_validate_paged_decode": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                                          _c_void_p, _i64, _i64, _c_void_p, _i64, _c_void_p,
                                          _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                          _i32, _c_void_p, _size_t]),
    "msgl_validate_store_kv_paged_decode": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64,
                                                   _c_void_p, _c_void_p, _i64, _i64, _c_void_p,
                                                   _c_void_p, _i64, _c_void_p, _i32, _c_void_p,
                                                   _i64, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                                   _i32, _i32, _i32, _f32, _i32, _c_void_p,
                                                   _size_t]),
    "msgl_validate_paged_extend": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                                          _c_void_p, _i64, _i64, _c_void_p, _i64, _c_void_p,
                                          _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                          _i32, _i32, _i32, _i32, _f32, _i32, _c_void_p,
                                          _size_t]),
    "msgl_validate_merge_states": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                          _i64, _i32, _i32, _i32]),
    "msgl_decode_graph_layout": (_i32, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_size_t)]),
    "msgl_decode_graph_create": (_i32, [_c_void_p, _c_void_p, _i64, _i64, _c_void_p, _i64, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _i32,
                                        _c_void_p, _size_t, ctypes.POINTER(_c_void_p)]),
    "msgl_decode_graph_run": (_i32, [_c_void_p, _i32, _c_void_p]),
    "msgl_decode_graph_bucket": (_i32, [_c_void_p, _i32]),
    "msgl_decode_graph_destroy": (None, [_c_void_p]),
}


class MsglError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        text = lib.msgl_status_string(status).decode()
        detail = lib.msgl_last_error().decode()
        super().__init__(f"{where}: {text} [{detail}]")
        self.status = status


def load(path: str | None = None):
    """Load libmsgl.so (built by ``__graft_entry__.build()``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("MSGL_LIBRARY", LIB_PATH)
    if not os.path.exists(path):
        raise RuntimeError(f"libmsgl not built: {path} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


@contextlib.contextmanager
def using_library(path: str):
    """Route the calls made inside the block through the library at ``path``
    (e.g. DEBUG_LIB_PATH, the debug-check build); the previous one afterwards."""
    global _lib
    saved = _lib
    _lib = None
    try:
        yield load(path)
    finally:
        _lib = saved


def _check(status: int, where: str) -> None:
    if status != MSGL_OK:
        raise MsglError(status, where)


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, dtype, name: str, dims=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {tuple(t.shape)}")


def _pool_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """Pool planes are [num_slots, Hkv, D] (heads and dims contiguous)."""
    _need(k_cache, torch.bfloat16, "k_cache", 3)
    _need(v_cache, torch.bfloat16, "v_cache", 3)
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    n, hkv, d = k_cache.shape
    if k_cache.stride(2) != 1 or k_cache.stride(1) != d:
        raise ValueError("pool rows must hold kv heads x head_dim contiguously")
    return n, hkv, d, k_cache.stride(0)


def version() -> int:
    return load().msgl_version()


class PlannedCall:
    """One validated, marshalled library call.

    ``plan_*`` functions check shapes and dtypes, allocate what the caller
    left out and fix every argument except the stream; ``run()`` then issues
    the C call alone (one ctypes call), e.g. once per layer of a model whose
    batch metadata is fixed for the step.  The tensors the plan refers to must
    stay alive and keep their storage; ``run()`` returns ``outputs``.
    """

    __slots__ = ("_fn", "_args", "_name", "outputs", "_keep")

    def __init__(self, fn, args, name, outputs, keep):
        self._fn, self._args, self._name = fn, tuple(args), name
        self.outputs, self._keep = outputs, keep

    def run(self, stream=None):
        st = self._fn(*self._args, _stream(stream))
        if st:
            _check(st, self._name)
        return self.outputs


# ---------------------------------------------------------------------------
# store_kv
# ---------------------------------------------------------------------------

def store_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
             v_new: torch.Tensor, out_loc: torch.Tensor, stream=None) -> None:
    """k_cache[out_loc[i]] = k_new[i] and likewise for V (in place)."""
    plan_store_kv(k_cache, v_cache, k_new, v_new, out_loc).run(stream)


def plan_store_kv(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                  v_new: torch.Tensor, out_loc: torch.Tensor) -> PlannedCall:
    """Planned form of :func:`store_kv`."""
    lib = load()
    if k_cache.dim() != 3 or k_new.dim() != 3:
        raise ValueError("k_cache [slots, Hkv, D] and k_new [n, Hkv, D] expected")
    if k_cache.dtype not in (torch.bfloat16, torch.float32) or k_new.dtype != k_cache.dtype \
            or v_cache.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype:
        raise TypeError("pool and new rows must share one dtype (bf16 or f32)")
    if out_loc.dtype not in (torch.int32, torch.int64):
        raise TypeError("out_loc must be int32 or int64")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new),
                    ("v_new", v_new), ("out_loc", out_loc)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    n_slots, hkv, d = k_cache.shape
    if tuple(k_new.shape[1:]) != (hkv, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch between pool planes and new rows")
    for t in (k_cache, v_cache, k_new, v_new):
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError("rows must hold kv heads x head_dim contiguously")
    if k_cache.stride(0) != v_cache.stride(0) or k_new.stride(0) != v_new.stride(0):
        raise ValueError("K and V planes must share row strides")
    if out_loc.dim() != 1 or out_loc.shape[0] != k_new.shape[0] or not out_loc.is_contiguous():
        raise ValueError("out_loc must be a contiguous [n] vector")
    args = (_ptr(k_cache), _ptr(v_cache), n_slots, k_cache.stride(0), _ptr(k_new), _ptr(v_new),
            k_new.stride(0), _ptr(out_loc), INDEX_I64 if out_loc.dtype == torch.int64 else INDEX_I32,
            k_new.shape[0], hkv, d, DTYPE_BF16 if k_cache.dtype == torch.bfloat16 else DTYPE_F32)
    return PlannedCall(lib.msgl_store_kv, args, "msgl_store_kv", None,
                       (k_cache, v_cache, k_new, v_new, out_loc))


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def paged_decode_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int,
                                max_seq_len: int, split_tokens: int = 0,
                                head_dim: int = 128) -> tuple[int, int]:
    """(bytes, split size used) for a decode call with these host sizes."""
    lib = load()
    s = _i32(0)
    n = lib.msgl_paged_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                             max_seq_len, split_tokens, ctypes.byref(s))
    return int(n), int(s.value)


def paged_extend_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int,
                                max_extend_len: int, max_kv_len: int,
                                head_dim: int = 128) -> int:
    """Bytes of the (optional) work-list workspace of an extend call."""
    lib = load()
    return int(lib.msgl_paged_extend_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                    max_extend_len, max_kv_len))


def alloc_workspace(nbytes: int, device=None) -> torch.Tensor | None:
    if nbytes <= 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device or "cuda")


def paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                 sm_scale: float, req_rows: torch.Tensor | None = None, page_size: int = 1,
                 split_tokens: int = 0, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, want_lse: bool = True,
                 workspace: torch.Tensor | None = None, stream=None):
    """Decode attention.  q [B, Hq, 128] bf16 (row stride free, heads contiguous).

    Returns ``(out [B, Hq, 128] bf16, lse [B, Hq] fp32 or None)``.
    """
    return plan_paged_decode(q, k_cache, v_cache, page_table, seq_lens, max_seq_len, sm_scale,
                             req_rows, page_size, split_tokens, out, lse, want_lse,
                             workspace).run(stream)


def plan_paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                      sm_scale: float, req_rows: torch.Tensor | None = None,
                      page_size: int = 1, split_tokens: int = 0,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      want_lse: bool = True,
                      workspace: torch.Tensor | None = None) -> PlannedCall:
    """Planned form of :func:`paged_decode`; ``run()`` returns ``(out, lse)``."""
    lib = load()
    d = _decode_args(q, k_cache, v_cache, page_table, seq_lens, max_seq_len, sm_scale, req_rows,
                     page_size, split_tokens, out, lse, want_lse, workspace)
    return PlannedCall(lib.msgl_paged_decode, d["args"], "msgl_paged_decode", d["outputs"],
                       d["keep"])


def store_kv_paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          k_new: torch.Tensor, v_new: torch.Tensor, out_loc: torch.Tensor,
                          page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                          sm_scale: float, req_rows: torch.Tensor | None = None,
                          page_size: int = 1, split_tokens: int = 0,
                          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                          want_lse: bool = True, workspace: torch.Tensor | None = None,
                          stream=None):
    """store_kv of one new row per request, then decode, in one launch.

    Row r of ``k_new`` / ``v_new`` [B, Hkv, 128] is request r's newest token;
    it goes to slot ``out_loc[r]``, which must be ``page_table[row_r,
    seq_lens[r] - 1]`` and no key of another request of the batch (a freshly
    allocated slot).  Returns ``(out, lse)`` like :func:`paged_decode`.
    """
    return plan_store_kv_paged_decode(q, k_cache, v_cache, k_new, v_new, out_loc, page_table,
                                      seq_lens, max_seq_len, sm_scale, req_rows, page_size,
                                      split_tokens, out, lse, want_lse, workspace).run(stream)


def plan_store_kv_paged_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               k_new: torch.Tensor, v_new: torch.Tensor, out_loc: torch.Tensor,
                               page_table: torch.Tensor, seq_lens: torch.Tensor,
                               max_seq_len: int, sm_scale: float,
                               req_rows: torch.Tensor | None = None, page_size: int = 1,
                               split_tokens: int = 0, out: torch.Tensor | None = None,
                               lse: torch.Tensor | None = None, want_lse: bool = True,
                               workspace: torch.Tensor | None = None) -> PlannedCall:
    """Planned form of :func:`store_kv_paged_decode`."""
    lib = load()
    d = _decode_args(q, k_cache, v_cache, page_table, seq_lens, max_seq_len, sm_scale, req_rows,
                     page_size, split_tokens, out, lse, want_lse, workspace)
    B, hkv, dim = q.shape[0], k_cache.shape[1], k_cache.shape[2]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, torch.bfloat16, name, 3)
        if tuple(t.shape) != (B, hkv, dim) or t.stride(2) != 1 or t.stride(1) != dim:
            raise ValueError(f"{name} must be [B, Hkv, D] with heads x dims contiguous")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must share a row stride")
    if out_loc.dtype not in (torch.int32, torch.int64) or not out_loc.is_cuda:
        raise TypeError("out_loc must be an int32 or int64 GPU tensor")
    if out_loc.dim() != 1 or out_loc.shape[0] != B or not out_loc.is_contiguous():
        raise ValueError("out_loc must be a contiguous [B] vector")
    a = d["args"]
    # (out, lse, q, q_stride, k, v, slots, cstride) + new rows + (page_table ...)
    args = (*a[:8], _ptr(k_new), _ptr(v_new), k_new.stride(0), _ptr(out_loc),
            INDEX_I64 if out_loc.dtype == torch.int64 else INDEX_I32, *a[8:])
    return PlannedCall(lib.msgl_store_kv_paged_decode, args, "msgl_store_kv_paged_decode",
                       d["outputs"], (*d["keep"], k_new, v_new, out_loc))


def store_kv_paged_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                  v_cache: torch.Tensor, k_new: torch.Tensor,
                                  v_new: torch.Tensor, out_loc: torch.Tensor,
                                  page_table: torch.Tensor, seq_lens: torch.Tensor,
                                  max_seq_len: int, sm_scale: float,
                                  req_rows: torch.Tensor | None = None, page_size: int = 1,
                                  split_tokens: int = 0, out: torch.Tensor | None = None,
                                  lse: torch.Tensor | None = None, want_lse: bool = True,
                                  stream=None):
    """:func:`store_kv_paged_decode` through the entry point that takes no
    workspace: its partial results live in the library's static device
    scratch (``MSGL_DECODE_SCRATCH_BYTES``), so no device memory is allocated
    for them.  Calls whose work overlaps on one GPU race on that scratch."""
    lib = load()
    d = _decode_args(q, k_cache, v_cache, page_table, seq_lens, max_seq_len, sm_scale, req_rows,
                     page_size, split_tokens, out, lse, want_lse, None, with_workspace=False)
    B, hkv, dim = q.shape[0], k_cache.shape[1], k_cache.shape[2]
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, torch.bfloat16, name, 3)
        if tuple(t.shape) != (B, hkv, dim) or t.stride(2) != 1 or t.stride(1) != dim:
            raise ValueError(f"{name} must be [B, Hkv, D] with heads x dims contiguous")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must share a row stride")
    if out_loc.dtype not in (torch.int32, torch.int64) or not out_loc.is_cuda:
        raise TypeError("out_loc must be an int32 or int64 GPU tensor")
    if out_loc.dim() != 1 or out_loc.shape[0] != B or not out_loc.is_contiguous():
        raise ValueError("out_loc must be a contiguous [B] vector")
    a = d["args"]
    # (out, lse, q, q_stride, k, v, slots, cstride) + new rows + (page_table ..
    # split_tokens), without the workspace pointer and size
    args = (*a[:8], _ptr(k_new), _ptr(v_new), k_new.stride(0), _ptr(out_loc),
            INDEX_I64 if out_loc.dtype == torch.int64 else INDEX_I32, *a[8:-2])
    return PlannedCall(lib.msgl_store_kv_paged_decode_noalloc, args,
                       "msgl_store_kv_paged_decode_noalloc", d["outputs"],
                       (*d["keep"], k_new, v_new, out_loc)).run(stream)


def _decode_args(q, k_cache, v_cache, page_table, seq_lens, max_seq_len, sm_scale, req_rows,
                 page_size, split_tokens, out, lse, want_lse, workspace, with_workspace=True):
    """Checks and marshals the arguments shared by the decode entry points."""
    _need(q, torch.bfloat16, "q", 3)
    n_slots, hkv, d, cstride = _pool_geometry(k_cache, v_cache)
    B, hq, dq = q.shape
    if dq != d or q.stride(2) != 1 or q.stride(1) != d:
        raise ValueError("q must be [B, Hq, D] with heads x dims contiguous")
    _need(page_table, torch.int32, "page_table", 2)
    _need(seq_lens, torch.int32, "seq_lens", 1)
    if page_table.stride(1) != 1:
        raise ValueError("page_table rows must be contiguous")
    if seq_lens.shape[0] != B or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be a contiguous [B] vector")
    if req_rows is not None:
        _need(req_rows, torch.int32, "req_rows", 1)
        if req_rows.shape[0] != B or not req_rows.is_contiguous():
            raise ValueError("req_rows must be a contiguous [B] vector")
    if out is None:
        out = torch.empty((B, hq, d), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", 3)
    if not out.is_contiguous() or tuple(out.shape) != (B, hq, d):
        raise ValueError("out must be a contiguous [B, Hq, D] tensor")
    if want_lse and lse is None:
        lse = torch.empty((B, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", 2)
        if not lse.is_contiguous() or tuple(lse.shape) != (B, hq):
            raise ValueError("lse must be a contiguous [B, Hq] tensor")
    need, _ = paged_decode_workspace_size(B, hq, hkv, max(1, max_seq_len), split_tokens, d)
    if workspace is None and need and with_workspace:
        workspace = alloc_workspace(need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(out), _ptr(lse), _ptr(q), q.stride(0), _ptr(k_cache), _ptr(v_cache), n_slots,
            cstride, _ptr(page_table), page_table.stride(0), _ptr(req_rows), _ptr(seq_lens), B, hq,
            hkv, d, page_size, max_seq_len, float(sm_scale), split_tokens, _ptr(workspace),
            ws_bytes)
    return {"args": args, "outputs": (out, lse),
            "keep": (q, k_cache, v_cache, page_table, seq_lens, req_rows, workspace)}


# ---------------------------------------------------------------------------
# extend
# ---------------------------------------------------------------------------

def paged_extend(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 page_table: torch.Tensor, prefix_lens: torch.Tensor,
                 extend_lens: torch.Tensor, q_offsets: torch.Tensor, max_extend_len: int,
                 max_kv_len: int, sm_scale: float, req_rows: torch.Tensor | None = None,
                 page_size: int = 1, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, want_lse: bool = True,
                 workspace: torch.Tensor | None = None, plan: bool = True, stream=None):
    """Causal extend.  q [T, Hq, 128] bf16; returns (out [T, Hq, 128], lse [T, Hq]).

    ``plan``: order the work longest first through a work-list workspace
    (``workspace`` if given, else one allocated here); ``plan=False`` passes
    no workspace.  The results are bit-identical either way.
    """
    return plan_paged_extend(q, k_cache, v_cache, page_table, prefix_lens, extend_lens,
                             q_offsets, max_extend_len, max_kv_len, sm_scale, req_rows,
                             page_size, out, lse, want_lse, workspace, plan).run(stream)


def plan_paged_extend(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      page_table: torch.Tensor, prefix_lens: torch.Tensor,
                      extend_lens: torch.Tensor, q_offsets: torch.Tensor, max_extend_len: int,
                      max_kv_len: int, sm_scale: float, req_rows: torch.Tensor | None = None,
                      page_size: int = 1, out: torch.Tensor | None = None,
                      lse: torch.Tensor | None = None, want_lse: bool = True,
                      workspace: torch.Tensor | None = None, plan: bool = True) -> PlannedCall:
    """Planned form of :func:`paged_extend`; ``run()`` returns ``(out, lse)``."""
    lib = load()
    _need(q, torch.bfloat16, "q", 3)
    n_slots, hkv, d, cstride = _pool_geometry(k_cache, v_cache)
    T, hq, dq = q.shape
    if dq != d or q.stride(2) != 1 or q.stride(1) != d:
        raise ValueError("q must be [T, Hq, D] with heads x dims contiguous")
    _need(page_table, torch.int32, "page_table", 2)
    B = extend_lens.shape[0]
    for name, t, n in (("prefix_lens", prefix_lens, B), ("extend_lens", extend_lens, B),
                       ("q_offsets", q_offsets, B + 1)):
        _need(t, torch.int32, name, 1)
        if t.shape[0] != n or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [{n}] vector")
    if req_rows is not None:
        _need(req_rows, torch.int32, "req_rows", 1)
        if req_rows.shape[0] != B or not req_rows.is_contiguous():
            raise ValueError("req_rows must be a contiguous [B] vector")
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, "out", 3)
    if not out.is_contiguous() or tuple(out.shape) != (T, hq, d):
        raise ValueError("out must be a contiguous [T, Hq, D] tensor")
    if want_lse and lse is None:
        lse = torch.empty((T, hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", 2)
        if not lse.is_contiguous() or tuple(lse.shape) != (T, hq):
            raise ValueError("lse must be a contiguous [T, Hq] tensor")
    if plan and workspace is None:
        workspace = alloc_workspace(
            paged_extend_workspace_size(B, hq, hkv, max_extend_len, max_kv_len, d), q.device)
    if not plan:
        workspace = None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(out), _ptr(lse), _ptr(q), q.stride(0), _ptr(k_cache), _ptr(v_cache), n_slots,
            cstride, _ptr(page_table), page_table.stride(0), _ptr(req_rows), _ptr(prefix_lens),
            _ptr(extend_lens), _ptr(q_offsets), B, hq, hkv, d, page_size, max_extend_len,
            max_kv_len, float(sm_scale), 1, _ptr(workspace), ws_bytes)
    return PlannedCall(lib.msgl_paged_extend, args, "msgl_paged_extend", (out, lse),
                       (q, k_cache, v_cache, page_table, prefix_lens, extend_lens, q_offsets,
                        req_rows, workspace))


# ---------------------------------------------------------------------------
# merge
# ---------------------------------------------------------------------------

def merge_states(part_out: torch.Tensor, part_lse: torch.Tensor,
                 out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, want_lse: bool = True, stream=None):
    """part_out [S, N, H, D] fp32, part_lse [S, N, H] fp32 -> (out [N, H, D], lse [N, H])."""
    lib = load()
    _need(part_out, torch.float32, "part_out", 4)
    _need(part_lse, torch.float32, "part_lse", 3)
    if not part_out.is_contiguous() or not part_lse.is_contiguous():
        raise ValueError("partials must be contiguous")
    S, N, H, D = part_out.shape
    if tuple(part_lse.shape) != (S, N, H):
        raise ValueError("part_lse must be [S, N, H]")
    if out is None:
        out = torch.empty((N, H, D), dtype=out_dtype, device=part_out.device)
    if want_lse and lse is None:
        lse = torch.empty((N, H), dtype=torch.float32, device=part_out.device)
    code = DTYPE_BF16 if out.dtype == torch.bfloat16 else DTYPE_F32
    st = lib.msgl_merge_states(_ptr(out), _ptr(lse), _ptr(part_out), _ptr(part_lse), S, N, H, D,
                               code, _stream(stream))
    _check(st, "msgl_merge_states")
    return out, lse


# ---------------------------------------------------------------------------
# embedding gather
# ---------------------------------------------------------------------------

def plan_embedding_gather(weights: torch.Tensor, ids: torch.Tensor, vocab_start: int = 0,
                          out: torch.Tensor | None = None) -> PlannedCall:
    """Planned form of :func:`embedding_gather`; ``run()`` returns ``out``."""
    lib = load()
    if weights.dim() != 2 or weights.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("weights must be a [rows, hidden] bf16 or fp32 tensor")
    if not weights.is_cuda or weights.stride(1) != 1:
        raise ValueError("weights must be a GPU tensor with contiguous rows")
    if ids.dim() != 1 or ids.dtype not in (torch.int32, torch.int64) or not ids.is_contiguous() \
            or not ids.is_cuda:
        raise TypeError("ids must be a contiguous [n] int32 / int64 GPU tensor")
    rows, hidden = weights.shape
    n = ids.shape[0]
    if out is None:
        out = torch.empty((n, hidden), dtype=weights.dtype, device=weights.device)
    if out.dtype != weights.dtype or tuple(out.shape) != (n, hidden) or out.stride(1) != 1:
        raise ValueError("out must be [n, hidden] of the table's dtype with contiguous rows")
    args = (_ptr(out), out.stride(0), _ptr(weights), rows, weights.stride(0), _ptr(ids),
            INDEX_I64 if ids.dtype == torch.int64 else INDEX_I32, n, int(vocab_start), hidden,
            DTYPE_BF16 if weights.dtype == torch.bfloat16 else DTYPE_F32)
    return PlannedCall(lib.msgl_embedding_gather, args, "msgl_embedding_gather", out,
                       (weights, ids))


def embedding_gather(weights: torch.Tensor, ids: torch.Tensor, vocab_start: int = 0,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """out[i] = weights[ids[i] - vocab_start], zeros for ids outside this shard."""
    return plan_embedding_gather(weights, ids, vocab_start, out).run(stream)


# ---------------------------------------------------------------------------
# attention-layer prologue: q/k RMSNorm + RoPE + store
# ---------------------------------------------------------------------------

def rope_cos_sin_cache(max_position: int, rotary_dim: int = 128, base: float = 1_000_000.0,
                       device=None, stream=None) -> torch.Tensor:
    """fp32 [max_position, rotary_dim] table: cos | sin of p * base^(-2i/rotary_dim)."""
    lib = load()
    cache = torch.empty((max_position, rotary_dim), dtype=torch.float32, device=device or "cuda")
    st = lib.msgl_rope_cos_sin_cache(_ptr(cache), max_position, rotary_dim, float(base),
                                     _stream(stream))
    _check(st, "msgl_rope_cos_sin_cache")
    return cache


def plan_qk_norm_rope_store(qkv: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            positions: torch.Tensor, cos_sin_cache: torch.Tensor,
                            out_loc: torch.Tensor, num_q_heads: int, num_kv_heads: int,
                            q_norm_weight: torch.Tensor | None = None,
                            k_norm_weight: torch.Tensor | None = None, eps: float = 1e-6,
                            q_out: torch.Tensor | None = None) -> PlannedCall:
    """Planned form of :func:`qk_norm_rope_store`; ``run()`` returns ``q_out``."""
    lib = load()
    n_slots, hkv, d, cstride = _pool_geometry(k_cache, v_cache)
    _need(qkv, torch.bfloat16, "qkv", 2)
    if hkv != num_kv_heads or qkv.shape[1] != (num_q_heads + 2 * num_kv_heads) * d \
            or qkv.stride(1) != 1:
        raise ValueError("qkv must be [n, (Hq + 2 Hkv) * D] with contiguous rows")
    n = qkv.shape[0]
    _need(positions, torch.int32, "positions", 1)
    _need(cos_sin_cache, torch.float32, "cos_sin_cache", 2)
    if positions.shape[0] != n or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous [n] vector")
    if cos_sin_cache.shape[1] != d or not cos_sin_cache.is_contiguous():
        raise ValueError("cos_sin_cache must be a contiguous [max_position, D] table")
    if out_loc.dim() != 1 or out_loc.shape[0] != n or out_loc.dtype not in (torch.int32, torch.int64) \
            or not out_loc.is_contiguous():
        raise ValueError("out_loc must be a contiguous [n] int32 / int64 vector")
    for name, w in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if w is not None:
            _need(w, torch.bfloat16, name, 1)
            if w.shape[0] != d or not w.is_contiguous():
                raise ValueError(f"{name} must be a contiguous [D] vector")
    if q_out is None:
        q_out = torch.empty((n, num_q_heads, d), dtype=torch.bfloat16, device=qkv.device)
    q_stride = q_out.stride(0)
    if q_out.dtype != torch.bfloat16 or q_out.shape[0] != n or q_out.stride(-1) != 1:
        raise ValueError("q_out must be bf16 [n, Hq, D] (or the qkv buffer itself)")
    args = (_ptr(q_out), q_stride, _ptr(k_cache), _ptr(v_cache), n_slots, cstride, _ptr(qkv),
            qkv.stride(0), _ptr(q_norm_weight), _ptr(k_norm_weight), float(eps), _ptr(positions),
            _ptr(cos_sin_cache), cos_sin_cache.shape[0], _ptr(out_loc),
            INDEX_I64 if out_loc.dtype == torch.int64 else INDEX_I32, n, num_q_heads,
            num_kv_heads, d)
    return PlannedCall(lib.msgl_qk_norm_rope_store, args, "msgl_qk_norm_rope_store", q_out,
                       (qkv, k_cache, v_cache, positions, cos_sin_cache, out_loc, q_norm_weight,
                        k_norm_weight))


def qk_norm_rope_store(qkv, k_cache, v_cache, positions, cos_sin_cache, out_loc, num_q_heads,
                       num_kv_heads, q_norm_weight=None, k_norm_weight=None, eps=1e-6,
                       q_out=None, stream=None) -> torch.Tensor:
    """q/k RMSNorm + RoPE of one layer's merged qkv; stores k, v into the pool at out_loc
    and returns the rotated q ([n, Hq, D] bf16, or ``q_out``)."""
    return plan_qk_norm_rope_store(qkv, k_cache, v_cache, positions, cos_sin_cache, out_loc,
                                   num_q_heads, num_kv_heads, q_norm_weight, k_norm_weight, eps,
                                   q_out).run(stream)


class DecodeGraph:
    """Graph-replayed decode step (``msgl_decode_graph_*``): padding +
    store_kv + paged_decode captured per batch size of the ladder [1, 2, 4,
    8, 16, ..., max_bs] over fixed buffers.  Write rows [0, batch) of ``q``,
    ``k_new``, ``v_new``, ``seq_lens``, ``req_rows``, ``out_loc`` (torch
    views of the buffer), call ``run(batch)``, read rows [0, batch) of
    ``out`` / ``lse``.  ``page_table[dummy_row, 0]`` must be
    ``sentinel_slot``, a slot no request owns.  ``fused_store``: capture the
    one-launch store + decode (``msgl_store_kv_paged_decode``), which needs
    each request's ``out_loc`` to be its own newest key and no other
    request's key."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                 num_q_heads: int, max_bs: int, max_seq_len: int, sm_scale: float,
                 dummy_row: int, sentinel_slot: int, page_size: int = 1,
                 fused_store: bool = False):
        lib = load()
        _need(k_cache, torch.bfloat16, "k_cache", 3)
        _need(page_table, torch.int32, "page_table", 2)
        slots, hkv, d = k_cache.shape
        off = (_size_t * 10)()
        _check(lib.msgl_decode_graph_layout(max_bs, num_q_heads, hkv, d, max_seq_len, off),
               "msgl_decode_graph_layout")
        self.buffer = torch.zeros(int(off[9]), dtype=torch.uint8, device=k_cache.device)
        self._keep = (k_cache, v_cache, page_table)

        def view(i, dtype, shape):
            n = 1
            for x in shape:
                n *= x
            nbytes = n * torch.empty((), dtype=dtype).element_size()
            return self.buffer[off[i]:off[i] + nbytes].view(dtype).view(*shape)

        self.q = view(0, torch.bfloat16, (max_bs, num_q_heads, d))
        self.k_new = view(1, torch.bfloat16, (max_bs, hkv, d))
        self.v_new = view(2, torch.bfloat16, (max_bs, hkv, d))
        self.out = view(3, torch.bfloat16, (max_bs, num_q_heads, d))
        self.lse = view(4, torch.float32, (max_bs, num_q_heads))
        self.seq_lens = view(5, torch.int32, (max_bs,))
        self.req_rows = view(6, torch.int32, (max_bs,))
        self.out_loc = view(7, torch.int32, (max_bs,))
        h = _c_void_p()
        _check(lib.msgl_decode_graph_create(
            k_cache.data_ptr(), v_cache.data_ptr(), slots, k_cache.stride(0),
            page_table.data_ptr(), page_table.stride(0), num_q_heads, hkv, d, page_size, max_bs,
            max_seq_len, sm_scale, dummy_row, sentinel_slot, 1 if fused_store else 0,
            self.buffer.data_ptr(),
            self.buffer.numel(), ctypes.byref(h)), "msgl_decode_graph_create")
        self._h = h
        self.max_bs = max_bs

    def bucket(self, batch: int) -> int:
        return int(load().msgl_decode_graph_bucket(self._h, batch))

    def run(self, batch: int, stream=None):
        _check(load().msgl_decode_graph_run(self._h, batch, _stream(stream)), "msgl_decode_graph_run")
        return self.out[:batch], self.lse[:batch]

    def close(self):
        if getattr(self, "_h", None):
            load().msgl_decode_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
