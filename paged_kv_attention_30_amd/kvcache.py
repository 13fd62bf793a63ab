"""ctypes binding of the host KV cache manager (``include/msgl_kvcache.h``).

Argument marshalling only: every operation runs in ``libmsgl.so``'s C++.
Token ids and lengths go in as numpy int32 / int64 arrays; the page table
comes back as a numpy view of the manager's host array (valid while the
manager lives).
"""

from __future__ import annotations

import ctypes

import numpy as np

from .binding import load

_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_VP = ctypes.c_void_p

_SIGS = {
    "msgl_kvc_create": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.POINTER(_VP)]),
    "msgl_kvc_destroy": (None, [_VP]),
    "msgl_kvc_page_table": (_I32P, [_VP]),
    "msgl_kvc_alloc_row": (ctypes.c_int, [_VP, _I32P]),
    "msgl_kvc_free_row": (ctypes.c_int, [_VP, ctypes.c_int32]),
    "msgl_kvc_match": (ctypes.c_int, [_VP, _I32P, ctypes.c_int64, ctypes.c_int32, _I64P, _I64P]),
    "msgl_kvc_lock": (ctypes.c_int, [_VP, ctypes.c_int64, ctypes.c_int32]),
    "msgl_kvc_allocate": (ctypes.c_int, [_VP, ctypes.c_int32, _I32P, _I64P, _I64P]),
    "msgl_kvc_cache_req": (ctypes.c_int, [_VP, ctypes.c_int32, _I32P, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int32, _I64P, _I64P]),
    "msgl_kvc_release": (ctypes.c_int, [_VP, ctypes.c_int32, ctypes.c_int64]),
    "msgl_kvc_evict": (ctypes.c_int, [_VP, ctypes.c_int64, _I64P]),
    "msgl_kvc_stats": (ctypes.c_int, [_VP, _I64P, ctypes.c_int32]),
    "msgl_kvc_free_list": (ctypes.c_int64, [_VP, _I32P, ctypes.c_int64]),
    "msgl_kvc_row_len": (ctypes.c_int64, [_VP, ctypes.c_int32]),
    "msgl_kvc_handle_len": (ctypes.c_int64, [_VP, ctypes.c_int64]),
    "msgl_compare_key": (ctypes.c_int64, [_I32P, ctypes.c_int64, _I32P, ctypes.c_int64]),
}

KVC_OK, KVC_ERR_ARG, KVC_ERR_FULL, KVC_ERR_STATE, KVC_ERR_NOMEM = 0, -1, -2, -3, -4


def _lib():
    lib = load()
    if not getattr(lib, "_msgl_kvc_sigs", False):
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        lib._msgl_kvc_sigs = True
    return lib


def _ids(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p32(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def compare_key(a, b) -> int:
    a, b = _ids(a), _ids(b)
    return int(_lib().msgl_compare_key(_p32(a), len(a), _p32(b), len(b)))


class KVCache:
    """Page allocator + radix prefix cache; methods return the C status
    (0 = ok) first, then their results."""

    def __init__(self, num_slots: int, page_size: int, max_rows: int, max_len: int):
        self._lib = _lib()
        h = _VP()
        st = self._lib.msgl_kvc_create(num_slots, page_size, max_rows, max_len, ctypes.byref(h))
        if st != KVC_OK:
            raise ValueError(f"msgl_kvc_create failed: status {st}")
        self._h = h
        self.page_size, self.max_rows, self.max_len = page_size, max_rows, max_len
        ptr = self._lib.msgl_kvc_page_table(self._h)
        self.page_table = np.ctypeslib.as_array(ptr, shape=(max_rows, max_len))

    def close(self):
        if self._h:
            self._lib.msgl_kvc_destroy(self._h)
            self._h = None
            self.page_table = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_row(self):
        r = ctypes.c_int32(-1)
        st = self._lib.msgl_kvc_alloc_row(self._h, ctypes.byref(r))
        return st, (r.value if st == KVC_OK else None)

    def free_row(self, row: int) -> int:
        return self._lib.msgl_kvc_free_row(self._h, row)

    def match(self, ids, row: int = -1):
        a = _ids(ids)
        cl, hd = ctypes.c_int64(0), ctypes.c_int64(0)
        st = self._lib.msgl_kvc_match(self._h, _p32(a), len(a), row, ctypes.byref(cl), ctypes.byref(hd))
        return st, cl.value, hd.value

    def lock(self, handle: int, delta: int) -> int:
        return self._lib.msgl_kvc_lock(self._h, handle, delta)

    def allocate(self, rows, cached_lens, device_lens) -> int:
        r = _ids(rows)
        c = np.ascontiguousarray(np.asarray(cached_lens, dtype=np.int64))
        d = np.ascontiguousarray(np.asarray(device_lens, dtype=np.int64))
        return self._lib.msgl_kvc_allocate(self._h, len(r), _p32(r), c.ctypes.data_as(_I64P),
                                           d.ctypes.data_as(_I64P))

    def cache_req(self, row: int, ids, cached_len: int, old_handle: int, finished: bool):
        a = _ids(ids)
        nh, nl = ctypes.c_int64(0), ctypes.c_int64(0)
        st = self._lib.msgl_kvc_cache_req(self._h, row, _p32(a), cached_len, old_handle,
                                          1 if finished else 0, ctypes.byref(nh), ctypes.byref(nl))
        return st, nh.value, nl.value

    def release(self, row: int, handle: int) -> int:
        return self._lib.msgl_kvc_release(self._h, row, handle)

    def evict(self, pages: int):
        f = ctypes.c_int64(0)
        st = self._lib.msgl_kvc_evict(self._h, pages, ctypes.byref(f))
        return st, f.value

    def stats(self) -> list[int]:
        out = (ctypes.c_int64 * 6)()
        st = self._lib.msgl_kvc_stats(self._h, out, 6)
        if st != KVC_OK:
            raise RuntimeError(f"msgl_kvc_stats: status {st}")
        return list(out)

    def free_list(self) -> np.ndarray:
        n = self._lib.msgl_kvc_free_list(self._h, None, 0)
        out = np.zeros(max(n, 0), dtype=np.int32)
        if n > 0:
            self._lib.msgl_kvc_free_list(self._h, _p32(out), n)
        return out

    def row_len(self, row: int) -> int:
        return int(self._lib.msgl_kvc_row_len(self._h, row))

    def handle_len(self, handle: int) -> int:
        return int(self._lib.msgl_kvc_handle_len(self._h, handle))
