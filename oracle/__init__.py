"""CPU oracle of the paged KV-cache write path (numpy front end over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  It shares
no code with the GPU library.  See oracle.c for the definitions and their
sources.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from .build import LIBRARY, build_oracle

PAD_ID = -1

ORC_OK, ORC_E_ARG, ORC_E_QSL, ORC_E_RANGES, ORC_E_DUPLICATE = 0, 1, 2, 3, 4
FLAG_NUM_TOKENS, FLAG_COUNT, FLAG_BAD_BLOCK, FLAG_SLOT_OOB = 1, 2, 4, 8

_ERRORS = {ORC_E_ARG: "invalid argument", ORC_E_QSL: "query_start_loc not non-decreasing",
           ORC_E_RANGES: "range descriptors violate the precondition",
           ORC_E_DUPLICATE: "two tokens share a slot"}


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what}: {_ERRORS.get(code, code)}")
        self.code = code


_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    out = np.ascontiguousarray(a, dtype=dtype)
    return out


class Oracle:
    """Bindings to one compiled copy of oracle.c."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build_oracle(output=path)
        lib = ctypes.CDLL(path)
        lib.orc_slot_mapping_paged.argtypes = [_P, _I32, _P, _I64, _P, _I32, _P, _I32, _P, _P]
        lib.orc_slot_mapping_ranges.argtypes = [_P, _I32, _P, _I64, _P, _P, _P, _P, _I32, _I32,
                                                _P, _P]
        lib.orc_slot_mapping_paged_cp.argtypes = [_P, _I32, _P, _I64, _P, _I32, _P, _I32, _I32,
                                                  _I32, _I32, _P, _P]
        lib.orc_slot_mapping_ranges_cp.argtypes = [_P, _I32, _P, _I64, _P, _P, _P, _P, _I32, _I32,
                                                   _I32, _I32, _I32, _P, _P]
        lib.orc_map_to_kernel_blocks.argtypes = [_P, _P, _I32, _I32, _I32, _I32, _P, _I32, _P,
                                                 _P]
        lib.orc_map_ranges_to_kernel_blocks.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                                        _P, _P, _P, _P, _P]
        lib.orc_ranges_to_block_table.argtypes = [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P,
                                                  _I32, _P, _P]
        lib.orc_decode_attention.argtypes = [_P, _P, _P, _I64, _P, _P, _P, _I32, _I32, _I32,
                                             _I32, ctypes.c_double, _P, _P]
        lib.orc_decode_attention.restype = ctypes.c_int
        lib.orc_coord_n.argtypes = [_I64] * 5
        lib.orc_coord_n.restype = _I64
        lib.orc_coord_offset.argtypes = [_I64] * 6
        lib.orc_coord_offset.restype = _I64
        lib.orc_kv_write.argtypes = [_P, _I64, _I32, _P, _P, _I64, _I64, _I64, _I32, _I64, _P, _P,
                                     _I64, _I64, _P]
        for f in (lib.orc_slot_mapping_paged, lib.orc_slot_mapping_ranges,
                  lib.orc_slot_mapping_paged_cp, lib.orc_slot_mapping_ranges_cp,
                  lib.orc_map_to_kernel_blocks, lib.orc_map_ranges_to_kernel_blocks,
                  lib.orc_ranges_to_block_table, lib.orc_kv_write):
            f.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    @staticmethod
    def _check(rc: int, what: str):
        if rc != ORC_OK:
            raise OracleError(rc, what)

    # -- slot mapping ------------------------------------------------------
    def slot_mapping_paged(self, query_start_loc, num_reqs: int, positions, max_num_tokens: int,
                           block_table, num_blocks_per_req, block_size: int
                           ) -> Tuple[np.ndarray, int]:
        qsl = _c(query_start_loc, np.int32)
        pos = _c(positions, np.int64)
        bt = _c(block_table, np.int32)
        nb = None if num_blocks_per_req is None else _c(num_blocks_per_req, np.int32)
        out = np.empty(max_num_tokens, dtype=np.int64)
        flags = ctypes.c_uint32(0)
        stride = bt.shape[1] if bt.ndim == 2 else 0
        rc = self.lib.orc_slot_mapping_paged(_ptr(qsl), num_reqs, _ptr(pos), max_num_tokens,
                                             _ptr(bt), stride, _ptr(nb), block_size, _ptr(out),
                                             ctypes.byref(flags))
        self._check(rc, "slot_mapping_paged")
        return out, flags.value

    def slot_mapping_ranges(self, query_start_loc, num_reqs: int, positions, max_num_tokens: int,
                            range_start, range_len, range_cum, num_ranges, block_size: int
                            ) -> Tuple[np.ndarray, int]:
        qsl = _c(query_start_loc, np.int32)
        pos = _c(positions, np.int64)
        rs, rl, rc_ = (_c(a, np.int32) for a in (range_start, range_len, range_cum))
        nr = _c(num_ranges, np.int32)
        out = np.empty(max_num_tokens, dtype=np.int64)
        flags = ctypes.c_uint32(0)
        rc = self.lib.orc_slot_mapping_ranges(_ptr(qsl), num_reqs, _ptr(pos), max_num_tokens,
                                              _ptr(rs), _ptr(rl), _ptr(rc_), _ptr(nr),
                                              rs.shape[1], block_size, _ptr(out),
                                              ctypes.byref(flags))
        self._check(rc, "slot_mapping_ranges")
        return out, flags.value

    # -- context-parallel slot mapping ---------------------------------------
    def slot_mapping_paged_cp(self, query_start_loc, num_reqs: int, positions,
                              max_num_tokens: int, block_table, num_blocks_per_req,
                              block_size: int, cp_world_size: int, cp_rank: int,
                              cp_interleave_size: int) -> Tuple[np.ndarray, int]:
        qsl = _c(query_start_loc, np.int32)
        pos = _c(positions, np.int64)
        bt = _c(block_table, np.int32)
        nb = None if num_blocks_per_req is None else _c(num_blocks_per_req, np.int32)
        out = np.empty(max_num_tokens, dtype=np.int64)
        flags = ctypes.c_uint32(0)
        stride = bt.shape[1] if bt.ndim == 2 else 0
        rc = self.lib.orc_slot_mapping_paged_cp(_ptr(qsl), num_reqs, _ptr(pos), max_num_tokens,
                                                _ptr(bt), stride, _ptr(nb), block_size,
                                                cp_world_size, cp_rank, cp_interleave_size,
                                                _ptr(out), ctypes.byref(flags))
        self._check(rc, "slot_mapping_paged_cp")
        return out, flags.value

    def slot_mapping_ranges_cp(self, query_start_loc, num_reqs: int, positions,
                               max_num_tokens: int, range_start, range_len, range_cum,
                               num_ranges, block_size: int, cp_world_size: int, cp_rank: int,
                               cp_interleave_size: int) -> Tuple[np.ndarray, int]:
        qsl = _c(query_start_loc, np.int32)
        pos = _c(positions, np.int64)
        rs, rl, rc_ = (_c(a, np.int32) for a in (range_start, range_len, range_cum))
        nr = _c(num_ranges, np.int32)
        out = np.empty(max_num_tokens, dtype=np.int64)
        flags = ctypes.c_uint32(0)
        rc = self.lib.orc_slot_mapping_ranges_cp(_ptr(qsl), num_reqs, _ptr(pos), max_num_tokens,
                                                 _ptr(rs), _ptr(rl), _ptr(rc_), _ptr(nr),
                                                 rs.shape[1], block_size, cp_world_size, cp_rank,
                                                 cp_interleave_size, _ptr(out),
                                                 ctypes.byref(flags))
        self._check(rc, "slot_mapping_ranges_cp")
        return out, flags.value

    # -- manager -> kernel block expansion --------------------------------
    def map_to_kernel_blocks(self, ids, counts, block_size: int, kernel_block_size: int,
                             out_stride: Optional[int] = None, with_counts: bool = False):
        """(table, flags), or (table, counts, flags) with with_counts."""
        a = _c(ids, np.int32)
        cnt = None if counts is None else _c(counts, np.int32)
        rows, in_stride = a.shape
        k = block_size // kernel_block_size if kernel_block_size > 0 else 0
        if out_stride is None:
            out_stride = in_stride * max(k, 1)
        out = np.empty((rows, out_stride), dtype=np.int32)
        counts_out = np.empty(rows, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        rc = self.lib.orc_map_to_kernel_blocks(_ptr(a), _ptr(cnt), rows, in_stride, block_size,
                                               kernel_block_size, _ptr(out), out_stride,
                                               _ptr(counts_out), ctypes.byref(flags))
        self._check(rc, "map_to_kernel_blocks")
        if with_counts:
            return out, counts_out, flags.value
        return out, flags.value

    def map_ranges_to_kernel_blocks(self, range_start, range_len, range_cum, num_ranges,
                                    block_size: int, kernel_block_size: int):
        rs, rl, rc_ = (_c(a, np.int32) for a in (range_start, range_len, range_cum))
        nr = _c(num_ranges, np.int32)
        rows, stride = rs.shape
        o_s, o_l, o_c = (np.empty((rows, stride), dtype=np.int32) for _ in range(3))
        o_n = np.empty(rows, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        rc = self.lib.orc_map_ranges_to_kernel_blocks(_ptr(rs), _ptr(rl), _ptr(rc_), _ptr(nr),
                                                      rows, stride, block_size, kernel_block_size,
                                                      _ptr(o_s), _ptr(o_l), _ptr(o_c), _ptr(o_n),
                                                      ctypes.byref(flags))
        self._check(rc, "map_ranges_to_kernel_blocks")
        return (o_s, o_l, o_c, o_n), flags.value

    def ranges_to_block_table(self, range_start, range_len, range_cum, num_ranges,
                              block_size: int, kernel_block_size: int, out_stride: int
                              ) -> Tuple[np.ndarray, np.ndarray, int]:
        """Block table [rows][out_stride] (kernel block ids) and per-row counts."""
        rs, rl, rc_ = (_c(a, np.int32) for a in (range_start, range_len, range_cum))
        nr = _c(num_ranges, np.int32)
        rows, stride = rs.shape
        out = np.empty((rows, out_stride), dtype=np.int32)
        counts = np.empty(rows, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        rc = self.lib.orc_ranges_to_block_table(_ptr(rs), _ptr(rl), _ptr(rc_), _ptr(nr), rows,
                                                stride, block_size, kernel_block_size, _ptr(out),
                                                out_stride, _ptr(counts), ctypes.byref(flags))
        self._check(rc, "ranges_to_block_table")
        return out, counts, flags.value

    # -- decode attention over the paged cache -------------------------------
    def decode_attention(self, q, k_cache, v_cache, slots_per_req, reqs, num_q_heads: int,
                         num_kv_heads: int, scale: float, with_lse: bool = False):
        """out[i][h][d] (float64) for requests reqs[i]; slots_per_req[i] lists the slots of
        positions 0, 1, ... of that request.  q: uint16 [R][Hq][D]; caches: uint16
        [rows][Hkv][D] (bf16 bit patterns).  with_lse: also return lse[i][h], the natural log
        of the softmax normalizer (-inf with no token)."""
        qq = _c(q, np.uint16)
        kc = _c(k_cache, np.uint16)
        vc = _c(v_cache, np.uint16)
        head_dim = qq.shape[-1]
        rows = kc.shape[0]
        slots = np.ascontiguousarray(np.concatenate([np.asarray(s, np.int64) for s in
                                                     slots_per_req] or [np.zeros(0, np.int64)]))
        begin = np.zeros(len(slots_per_req) + 1, np.int64)
        begin[1:] = np.cumsum([len(s) for s in slots_per_req])
        rq = _c(reqs, np.int32)
        out = np.zeros((len(rq), num_q_heads, head_dim), np.float64)
        lse = np.zeros((len(rq), num_q_heads), np.float64) if with_lse else None
        rc = self.lib.orc_decode_attention(_ptr(qq), _ptr(kc), _ptr(vc), rows, _ptr(slots),
                                           _ptr(begin), _ptr(rq), len(rq), num_q_heads,
                                           num_kv_heads, head_dim, float(scale), _ptr(out),
                                           _ptr(lse))
        self._check(rc, "decode_attention")
        return (out, lse) if with_lse else out

    # -- coordinate form ---------------------------------------------------
    def coord_n(self, layer, block, token, num_blocks, block_size) -> int:
        return int(self.lib.orc_coord_n(layer, block, token, num_blocks, block_size))

    def coord_offset(self, layer, block, token, num_blocks, block_size, bytes_per_token) -> int:
        return int(self.lib.orc_coord_offset(layer, block, token, num_blocks, block_size,
                                             bytes_per_token))

    # -- K/V scatter -------------------------------------------------------
    def kv_write(self, slot_mapping, key: np.ndarray, value: np.ndarray, num_blocks: int,
                 block_size: int, k_window: np.ndarray, v_window: np.ndarray,
                 row_begin: int = 0) -> int:
        """Write K/V rows into host windows of the caches; returns the flag bits.

        key, value: [num_layers, max_num_tokens, row] arrays (any dtype, C order).
        k_window, v_window: C-ordered arrays holding rows [row_begin, row_begin + n)
        of the [num_layers * num_blocks * block_size] cache row space.
        """
        sm = _c(slot_mapping, np.int64)
        if not (key.flags.c_contiguous and value.flags.c_contiguous):
            raise ValueError("key/value must be C-contiguous")
        if key.shape != value.shape or key.ndim != 3:
            raise ValueError("key/value must be [layers, tokens, row] and alike")
        layers, m, _ = key.shape
        bpt = key.strides[1]
        if not (k_window.flags.c_contiguous and v_window.flags.c_contiguous):
            raise ValueError("windows must be C-contiguous")
        if k_window.nbytes != v_window.nbytes or k_window.nbytes % bpt:
            raise ValueError("window size must be a whole number of rows")
        if sm.shape[0] != m:
            raise ValueError("slot_mapping length must equal the token dimension")
        flags = ctypes.c_uint32(0)
        rc = self.lib.orc_kv_write(_ptr(sm), m, layers, _ptr(key), _ptr(value), key.strides[0],
                                   key.strides[1], num_blocks, block_size, bpt, _ptr(k_window),
                                   _ptr(v_window), row_begin, k_window.nbytes // bpt,
                                   ctypes.byref(flags))
        self._check(rc, "kv_write")
        return flags.value


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle compiled from oracle/oracle.c (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
