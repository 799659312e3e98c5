"""Python binding of the contiguous-range allocator in libkvw.so (include/kvw_alloc.h).

Argument marshalling only: every operation runs in the native library.
Mutating methods return the kvw status code (0 = OK), as the C calls do;
exports raise KvwError on failure.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .kvw import KvwError, library

_P, _I32, _I64, _U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64


class kvw_alloc_stats(ctypes.Structure):
    _fields_ = [("usable_blocks", _I64), ("free_blocks", _I64), ("cache_only_blocks", _I64),
                ("free_runs", _I64), ("extents", _I64), ("cache_entries", _I64)]


_SIGS = {
    "kvw_alloc_create": [_I64, _I32, _I64, _I32, ctypes.POINTER(_P)],
    "kvw_alloc_extend": [_P, _I32, _I64],
    "kvw_alloc_release": [_P, _I32],
    "kvw_alloc_cache_insert": [_P, _U64, _I32, _I64, _I64],
    "kvw_alloc_cache_acquire": [_P, _U64, _I32],
    "kvw_alloc_cache_evict": [_P, _I64, ctypes.POINTER(_I64)],
    "kvw_alloc_ranges": [_P, _P, _I32, _I32, _P, _P, _P, _P],
    "kvw_alloc_block_table": [_P, _P, _I32, _I32, _P, _P],
    "kvw_alloc_row_extents": [_P, _I32, _I32, _P, _P, ctypes.POINTER(_I32)],
    "kvw_alloc_free_runs": [_P, _I64, _P, _P, ctypes.POINTER(_I64)],
    "kvw_alloc_lru": [_P, _I64, _P, _P, ctypes.POINTER(_I64)],
    "kvw_alloc_get_stats": [_P, ctypes.POINTER(kvw_alloc_stats)],
    "kvw_coord_offset": [_I64, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.POINTER(_I64)],
}
_bound = None


def _lib():
    global _bound
    if _bound is None:
        lib = library()
        for name, argtypes in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
        lib.kvw_alloc_destroy.argtypes = [_P]
        lib.kvw_alloc_destroy.restype = None
        _bound = lib
    return _bound


def _raise(status: int):
    if status != 0:
        raise KvwError(status, _lib().kvw_last_error().decode(errors="replace"))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


def kvw_coord_offset(layer, block, token, num_layers, num_blocks, block_size,
                     bytes_per_token) -> int:
    out = _I64(0)
    _raise(_lib().kvw_coord_offset(layer, block, token, num_layers, num_blocks, block_size,
                                   bytes_per_token, ctypes.byref(out)))
    return out.value


class RangeAllocator:
    """One native allocator (kvw_alloc_create ... kvw_alloc_destroy)."""

    def __init__(self, num_blocks: int, alignment: int = 1, first_block: int = 1,
                 max_rows: int = 256):
        self._h = _P()
        _raise(_lib().kvw_alloc_create(num_blocks, alignment, first_block, max_rows,
                                       ctypes.byref(self._h)))
        self.max_rows = max_rows
        self.alignment = alignment

    def close(self):
        if self._h:
            _lib().kvw_alloc_destroy(self._h)
            self._h = _P()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- operations (status codes) ----------------------------------------------
    def extend(self, row: int, n: int) -> int:
        return _lib().kvw_alloc_extend(self._h, row, n)

    def release(self, row: int) -> int:
        return _lib().kvw_alloc_release(self._h, row)

    def cache_insert(self, key: int, row: int, first: int, count: int) -> int:
        return _lib().kvw_alloc_cache_insert(self._h, key, row, first, count)

    def cache_acquire(self, key: int, row: int) -> int:
        return _lib().kvw_alloc_cache_acquire(self._h, key, row)

    def cache_evict(self, max_extents: int) -> Tuple[int, int]:
        k = _I64(0)
        st = _lib().kvw_alloc_cache_evict(self._h, max_extents, ctypes.byref(k))
        return st, k.value

    # -- views ----------------------------------------------------------------
    def row_extents(self, row: int) -> List[Tuple[int, int]]:
        n = _I32(0)
        _raise(_lib().kvw_alloc_row_extents(self._h, row, 0, None, None, ctypes.byref(n)))
        s = np.zeros(max(n.value, 1), np.int64)
        ln = np.zeros_like(s)
        _raise(_lib().kvw_alloc_row_extents(self._h, row, n.value, _ptr(s), _ptr(ln),
                                            ctypes.byref(n)))
        return [(int(a), int(b)) for a, b in zip(s[:n.value], ln[:n.value])]

    def ranges(self, rows: Sequence[int], range_stride: int):
        """(start, len, cum, num_ranges) arrays for rows, as the GPU calls take them."""
        r = np.ascontiguousarray(rows, dtype=np.int32)
        st, ln, cm = (np.zeros((len(r), range_stride), np.int32) for _ in range(3))
        nr = np.zeros(len(r), np.int32)
        _raise(_lib().kvw_alloc_ranges(self._h, _ptr(r), len(r), range_stride, _ptr(st),
                                       _ptr(ln), _ptr(cm), _ptr(nr)))
        return st, ln, cm, nr

    def block_table(self, rows: Sequence[int], stride: int):
        r = np.ascontiguousarray(rows, dtype=np.int32)
        t = np.zeros((len(r), stride), np.int32)
        c = np.zeros(len(r), np.int32)
        _raise(_lib().kvw_alloc_block_table(self._h, _ptr(r), len(r), stride, _ptr(t), _ptr(c)))
        return t, c

    def row_ranges(self, row: int) -> List[Tuple[int, int, int]]:
        n = max(1, len(self.row_extents(row)))
        st, ln, cm, nr = self.ranges([row], n)
        return [(int(st[0, i]), int(ln[0, i]), int(cm[0, i])) for i in range(int(nr[0]))]

    def free_runs(self) -> List[Tuple[int, int]]:
        n = _I64(0)
        _raise(_lib().kvw_alloc_free_runs(self._h, 0, None, None, ctypes.byref(n)))
        s = np.zeros(max(n.value, 1), np.int64)
        ln = np.zeros_like(s)
        _raise(_lib().kvw_alloc_free_runs(self._h, n.value, _ptr(s), _ptr(ln), ctypes.byref(n)))
        return [(int(a), int(b)) for a, b in zip(s[:n.value], ln[:n.value])]

    def lru_extents(self) -> List[Tuple[int, int]]:
        n = _I64(0)
        _raise(_lib().kvw_alloc_lru(self._h, 0, None, None, ctypes.byref(n)))
        s = np.zeros(max(n.value, 1), np.int64)
        ln = np.zeros_like(s)
        _raise(_lib().kvw_alloc_lru(self._h, n.value, _ptr(s), _ptr(ln), ctypes.byref(n)))
        return [(int(a), int(b)) for a, b in zip(s[:n.value], ln[:n.value])]

    def lru_starts(self) -> List[int]:
        return [s for s, _ in self.lru_extents()]

    def stats(self) -> Dict[str, int]:
        out = kvw_alloc_stats()
        _raise(_lib().kvw_alloc_get_stats(self._h, ctypes.byref(out)))
        return {name: int(getattr(out, name)) for name, _ in kvw_alloc_stats._fields_}
