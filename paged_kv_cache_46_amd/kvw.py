"""Python binding of libkvw.so (include/kvw.h): argument marshalling only.

Every function has the name of its C entry point and takes PyTorch tensors
that live on the GPU; PyTorch supplies device memory and streams, the
library's HIP kernels do all the work.  There is no fallback: if libkvw.so
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build import LIBRARY

KVW_ABI_VERSION = 7
KVW_PAD_ID = -1
KVW_MAX_RANGE_STRIDE = 65536
(KVW_OK, KVW_ERR_INVALID_ARG, KVW_ERR_UNSUPPORTED, KVW_ERR_RANGE_CAP, KVW_ERR_HIP,
 KVW_ERR_NO_SPACE, KVW_ERR_NOT_FOUND) = range(7)
KVW_FLAG_NUM_TOKENS, KVW_FLAG_COUNT, KVW_FLAG_BAD_BLOCK, KVW_FLAG_SLOT_OOB = 1, 2, 4, 8
KVW_SLOTS_PRECOMPUTED, KVW_SLOTS_PAGED, KVW_SLOTS_RANGES = 0, 1, 2
KVW_SCHEDULE_AUTO, KVW_SCHEDULE_TWO_KERNELS, KVW_SCHEDULE_ONE_KERNEL = 0, 1, 2
KVW_TWO_KERNEL_MIN_ROWS = 65536


class KvwError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvw status {status}: {message}")
        self.status = status


_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


class kvw_kv_write_args(ctypes.Structure):
    _fields_ = [
        ("mode", _I32), ("num_reqs", _I32),
        ("query_start_loc", _P), ("positions", _P), ("max_num_tokens", _I64),
        ("slot_mapping_in", _P), ("slot_mapping_out", _P),
        ("block_table", _P), ("num_blocks_per_req", _P),
        ("block_table_stride", _I32), ("range_stride", _I32),
        ("range_start", _P), ("range_len", _P), ("range_cum", _P), ("num_ranges", _P),
        ("block_size", _I32), ("num_layers", _I32), ("num_blocks", _I64),
        ("key", _P), ("value", _P), ("kv_layer_stride", _I64), ("kv_token_stride", _I64),
        ("k_cache", _P), ("v_cache", _P), ("bytes_per_token", _I64),
        ("err_flag", _P), ("schedule", _I32),
        ("cp_world_size", _I32), ("cp_rank", _I32), ("cp_interleave_size", _I32),
        ("table_out", _P), ("table_counts_out", _P), ("table_out_stride", _I32),
        ("table_block_size", _I32),
    ]


class kvw_decode_args(ctypes.Structure):
    _fields_ = [
        ("mode", _I32), ("num_reqs", _I32), ("q", _P), ("context_lens", _P),
        ("max_context", _I32), ("block_size", _I32), ("block_table", _P),
        ("num_blocks_per_req", _P), ("block_table_stride", _I32), ("range_stride", _I32),
        ("range_start", _P), ("range_len", _P), ("range_cum", _P), ("num_ranges", _P),
        ("k_cache", _P), ("v_cache", _P), ("num_blocks", _I64), ("num_q_heads", _I32),
        ("num_kv_heads", _I32), ("head_dim", _I32), ("scale", ctypes.c_float), ("out", _P),
        ("workspace", _P), ("workspace_bytes", _I64), ("err_flag", _P),
        ("chunk_positions", _I32), ("cp_world_size", _I32), ("cp_rank", _I32),
        ("cp_interleave_size", _I32), ("lse_out", _P),
    ]


_lib = None


def library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libkvw.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_46_amd.build`"
                           " (or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    sigs = {
        "kvw_slot_mapping_paged": [_P, _I32, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32, _P,
                                   _P, _P],
        "kvw_slot_mapping_ranges": [_P, _I32, _P, _I64, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                    _I32, _P, _P, _P],
        "kvw_map_to_kernel_blocks": [_P, _P, _I32, _I32, _I32, _I32, _P, _I32, _P, _P],
        "kvw_map_ranges_to_kernel_blocks": [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P,
                                            _P, _P, _P],
        "kvw_ranges_to_block_table": [_P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _I32, _P, _P,
                                      _P],
        "kvw_kv_write": [ctypes.POINTER(kvw_kv_write_args), _P],
        "kvw_decode_attention": [ctypes.POINTER(kvw_decode_args), _P],
        "kvw_decode_attention_noalloc": [ctypes.POINTER(kvw_decode_args), _P],
        "kvw_decode_merge": [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P],
    }
    for name, argtypes in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = ctypes.c_int
    lib.kvw_abi_version.restype = _I32
    lib.kvw_last_error.restype = ctypes.c_char_p
    lib.kvw_kv_write_args_size.restype = ctypes.c_size_t
    lib.kvw_decode_args_size.restype = ctypes.c_size_t
    lib.kvw_decode_workspace_size.argtypes = [_I32, _I32, _I32, _I32]
    lib.kvw_decode_workspace_size.restype = _I64
    if lib.kvw_abi_version() != KVW_ABI_VERSION:
        raise RuntimeError(f"libkvw ABI {lib.kvw_abi_version()} != binding ABI {KVW_ABI_VERSION}")
    if lib.kvw_kv_write_args_size() != ctypes.sizeof(kvw_kv_write_args):
        raise RuntimeError("kvw_kv_write_args layout differs between library and binding")
    if lib.kvw_decode_args_size() != ctypes.sizeof(kvw_decode_args):
        raise RuntimeError("kvw_decode_args layout differs between library and binding")
    _lib = lib
    return lib


def _check(status: int):
    if status != KVW_OK:
        raise KvwError(status, library().kvw_last_error().decode(errors="replace"))


def _dev(t: Optional[torch.Tensor], dtype: torch.dtype, name: str, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _positions(positions, max_num_tokens) -> int:
    """The positions pointer, after checking that all max_num_tokens entries exist (the
    kernels read every one of them, padded tokens' included)."""
    ptr = _dev(positions, torch.int64, "positions")
    if positions.numel() < int(max_num_tokens):
        raise ValueError(f"positions holds {positions.numel()} entries, fewer than max_num_tokens "
                         f"({int(max_num_tokens)})")
    return ptr


def _stride(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else (int(t.shape[1]) if t.dim() == 2 else int(t.numel()))


def kvw_slot_mapping_paged(query_start_loc, num_reqs, positions, max_num_tokens, block_table,
                           num_blocks_per_req, block_size, slot_mapping, err_flag=None,
                           stream=None, *, cp_world_size=1, cp_rank=0, cp_interleave_size=1):
    """slot_mapping[t] = block_table[r][p // bs] * bs + p % bs (see include/kvw.h); with
    cp_world_size > 1 only this context-parallel rank's positions get slots."""
    _check(library().kvw_slot_mapping_paged(
        _dev(query_start_loc, torch.int32, "query_start_loc"), int(num_reqs),
        _positions(positions, max_num_tokens), int(max_num_tokens),
        _dev(block_table, torch.int32, "block_table", optional=True), _stride(block_table),
        _dev(num_blocks_per_req, torch.int32, "num_blocks_per_req", optional=True),
        int(block_size), int(cp_world_size), int(cp_rank), int(cp_interleave_size),
        _dev(slot_mapping, torch.int64, "slot_mapping"),
        _dev(err_flag, torch.int32, "err_flag", optional=True), _stream(stream)))


def kvw_slot_mapping_ranges(query_start_loc, num_reqs, positions, max_num_tokens, range_start,
                            range_len, range_cum, num_ranges, block_size, slot_mapping,
                            err_flag=None, stream=None, *, cp_world_size=1, cp_rank=0,
                            cp_interleave_size=1):
    """slot = (start + lb - cum) * bs + p % bs for the run holding lb (see include/kvw.h); with
    cp_world_size > 1 only this context-parallel rank's positions get slots."""
    _check(library().kvw_slot_mapping_ranges(
        _dev(query_start_loc, torch.int32, "query_start_loc"), int(num_reqs),
        _positions(positions, max_num_tokens), int(max_num_tokens),
        _dev(range_start, torch.int32, "range_start"), _dev(range_len, torch.int32, "range_len"),
        _dev(range_cum, torch.int32, "range_cum"), _dev(num_ranges, torch.int32, "num_ranges"),
        _stride(range_start), int(block_size), int(cp_world_size), int(cp_rank),
        int(cp_interleave_size), _dev(slot_mapping, torch.int64, "slot_mapping"),
        _dev(err_flag, torch.int32, "err_flag", optional=True), _stream(stream)))


def kvw_map_to_kernel_blocks(ids, counts, block_size, kernel_block_size, out, err_flag=None,
                             stream=None):
    """out[r][i*k+j] = ids[r][i]*k + j, k = block_size // kernel_block_size."""
    _check(library().kvw_map_to_kernel_blocks(
        _dev(ids, torch.int32, "ids"), _dev(counts, torch.int32, "counts", optional=True),
        int(ids.shape[0]), int(ids.shape[1]), int(block_size), int(kernel_block_size),
        _dev(out, torch.int32, "out"), int(out.shape[1]),
        _dev(err_flag, torch.int32, "err_flag", optional=True), _stream(stream)))


def kvw_map_ranges_to_kernel_blocks(range_start, range_len, range_cum, num_ranges, block_size,
                                    kernel_block_size, out_start, out_len, out_cum,
                                    out_num_ranges, err_flag=None, stream=None):
    """(start, len, cum) -> (start*k, len*k, cum*k) for each run of each row."""
    _check(library().kvw_map_ranges_to_kernel_blocks(
        _dev(range_start, torch.int32, "range_start"), _dev(range_len, torch.int32, "range_len"),
        _dev(range_cum, torch.int32, "range_cum"), _dev(num_ranges, torch.int32, "num_ranges"),
        int(range_start.shape[0]), int(range_start.shape[1]), int(block_size),
        int(kernel_block_size), _dev(out_start, torch.int32, "out_start"),
        _dev(out_len, torch.int32, "out_len"), _dev(out_cum, torch.int32, "out_cum"),
        _dev(out_num_ranges, torch.int32, "out_num_ranges"),
        _dev(err_flag, torch.int32, "err_flag", optional=True), _stream(stream)))


def kvw_ranges_to_block_table(range_start, range_len, range_cum, num_ranges, block_size,
                              kernel_block_size, block_table, num_blocks_per_req=None,
                              err_flag=None, stream=None):
    """Fill block_table [rows][stride] (kernel block ids) from the range descriptors."""
    _check(library().kvw_ranges_to_block_table(
        _dev(range_start, torch.int32, "range_start"), _dev(range_len, torch.int32, "range_len"),
        _dev(range_cum, torch.int32, "range_cum"), _dev(num_ranges, torch.int32, "num_ranges"),
        int(range_start.shape[0]), int(range_start.shape[1]), int(block_size),
        int(kernel_block_size), _dev(block_table, torch.int32, "block_table"),
        int(block_table.shape[1]),
        _dev(num_blocks_per_req, torch.int32, "num_blocks_per_req", optional=True),
        _dev(err_flag, torch.int32, "err_flag", optional=True), _stream(stream)))


def kvw_kv_write(*, mode, key, value, k_cache, v_cache, num_blocks, block_size,
                 max_num_tokens=None, slot_mapping_in=None, slot_mapping_out=None,
                 query_start_loc=None, num_reqs=0, positions=None, block_table=None,
                 num_blocks_per_req=None, range_start=None, range_len=None, range_cum=None,
                 num_ranges=None, err_flag=None, schedule=KVW_SCHEDULE_AUTO, stream=None,
                 cp_world_size=1, cp_rank=0, cp_interleave_size=1, table_out=None,
                 table_counts_out=None, table_block_size=None):
    """K/V scatter into the paged cache, optionally fused with the slot mapping.

    key, value: [num_layers, max_num_tokens, H, D] (or [max_num_tokens, H, D]) tensors of a
    2-byte dtype; their row stride gives bytes_per_token.  k_cache, v_cache: any contiguous
    tensors holding num_layers * num_blocks * block_size such rows.  With cp_world_size > 1
    the caches are this context-parallel rank's (block_size slots per block) and only its
    positions are written.  table_out (optional, [num_reqs, stride] int32) receives the
    attention side's block table at table_block_size, made in the same launch as the slots.
    """
    for name, t in (("key", key), ("value", value)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if key.shape != value.shape or key.dtype != value.dtype:
        raise ValueError("key and value must match in shape and dtype")
    kv = key if key.dim() == 4 else key.unsqueeze(0)
    if kv.dim() != 4:
        raise ValueError("key must be [layers, tokens, heads, head_dim] or [tokens, heads, head_dim]")
    layers, m = int(kv.shape[0]), int(kv.shape[1])
    esz = key.element_size()
    bpt = int(kv.shape[2] * kv.shape[3] * esz)
    if max_num_tokens is None:
        max_num_tokens = m
    if int(max_num_tokens) > m:
        raise ValueError("max_num_tokens exceeds the token rows of key/value")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        need = layers * int(num_blocks) * int(block_size) * bpt
        if t.numel() * t.element_size() < need:
            raise ValueError(f"{name} holds fewer than layers*num_blocks*block_size rows")
    a = kvw_kv_write_args()
    a.mode = int(mode)
    a.num_reqs = int(num_reqs)
    a.max_num_tokens = int(max_num_tokens)
    a.block_size = int(block_size)
    a.num_layers = layers
    a.num_blocks = int(num_blocks)
    a.key, a.value = key.data_ptr(), value.data_ptr()
    a.kv_layer_stride = int(kv.stride(0) * esz)
    a.kv_token_stride = int(kv.stride(1) * esz)
    a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    a.bytes_per_token = bpt
    a.err_flag = _dev(err_flag, torch.int32, "err_flag", optional=True)
    a.schedule = int(schedule)
    a.cp_world_size, a.cp_rank = int(cp_world_size), int(cp_rank)
    a.cp_interleave_size = int(cp_interleave_size)
    if table_out is not None:
        a.table_out = _dev(table_out, torch.int32, "table_out")
        a.table_out_stride = _stride(table_out)
        a.table_counts_out = _dev(table_counts_out, torch.int32, "table_counts_out", optional=True)
        a.table_block_size = int(table_block_size if table_block_size is not None else block_size)
    if mode == KVW_SLOTS_PRECOMPUTED:
        a.slot_mapping_in = _dev(slot_mapping_in, torch.int64, "slot_mapping_in")
    else:
        a.query_start_loc = _dev(query_start_loc, torch.int32, "query_start_loc")
        a.positions = _positions(positions, max_num_tokens)
        a.slot_mapping_out = _dev(slot_mapping_out, torch.int64, "slot_mapping_out", optional=True)
        if mode == KVW_SLOTS_PAGED:
            a.block_table = _dev(block_table, torch.int32, "block_table", optional=True)
            a.block_table_stride = _stride(block_table)
            a.num_blocks_per_req = _dev(num_blocks_per_req, torch.int32, "num_blocks_per_req",
                                        optional=True)
        elif mode == KVW_SLOTS_RANGES:
            a.range_start = _dev(range_start, torch.int32, "range_start")
            a.range_len = _dev(range_len, torch.int32, "range_len")
            a.range_cum = _dev(range_cum, torch.int32, "range_cum")
            a.num_ranges = _dev(num_ranges, torch.int32, "num_ranges")
            a.range_stride = _stride(range_start)
    _check(library().kvw_kv_write(ctypes.byref(a), _stream(stream)))


def kvw_decode_workspace_size(num_reqs, max_context, num_q_heads, head_dim=128) -> int:
    return int(library().kvw_decode_workspace_size(num_reqs, max_context, num_q_heads, head_dim))


def _decode_args(mode, q, k_cache, v_cache, context_lens, max_context, num_blocks, block_size,
                 out, block_table, num_blocks_per_req, range_start, range_len, range_cum,
                 num_ranges, scale, workspace, err_flag, chunk_positions, cp_world_size, cp_rank,
                 cp_interleave_size, lse_out):
    """kvw_decode_args for the decode-attention calls (workspace: a byte tensor or None)."""
    if q.dim() != 3 or k_cache.dim() != 3 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [R, Hq, D] and the caches [rows, Hkv, D]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() \
                or t.element_size() != 2:
            raise ValueError(f"{name} must be a contiguous GPU tensor of a 2-byte dtype")
    if out.shape != q.shape or out.dtype != torch.float32:
        raise ValueError("out must be float32 with q's shape")
    num_reqs, hq, d = (int(x) for x in q.shape)
    hkv = int(k_cache.shape[1])
    a = kvw_decode_args()
    a.mode, a.num_reqs = int(mode), num_reqs
    a.q = q.data_ptr()
    a.context_lens = _dev(context_lens, torch.int32, "context_lens")
    a.max_context, a.block_size = int(max_context), int(block_size)
    if mode == KVW_SLOTS_PAGED:
        a.block_table = _dev(block_table, torch.int32, "block_table", optional=True)
        a.block_table_stride = _stride(block_table)
        a.num_blocks_per_req = _dev(num_blocks_per_req, torch.int32, "num_blocks_per_req",
                                    optional=True)
    else:
        a.range_start = _dev(range_start, torch.int32, "range_start")
        a.range_len = _dev(range_len, torch.int32, "range_len")
        a.range_cum = _dev(range_cum, torch.int32, "range_cum")
        a.num_ranges = _dev(num_ranges, torch.int32, "num_ranges")
        a.range_stride = _stride(range_start)
    a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    a.num_blocks = int(num_blocks)
    a.num_q_heads, a.num_kv_heads, a.head_dim = hq, hkv, d
    a.scale = float(scale if scale is not None else d ** -0.5)
    a.out = out.data_ptr()
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.err_flag = _dev(err_flag, torch.int32, "err_flag", optional=True)
    a.chunk_positions = int(chunk_positions)
    a.cp_world_size, a.cp_rank = int(cp_world_size), int(cp_rank)
    a.cp_interleave_size = int(cp_interleave_size)
    if lse_out is not None and (lse_out.dtype != torch.float32 or tuple(lse_out.shape) != (num_reqs, hq)):
        raise ValueError("lse_out must be float32 [num_reqs, num_q_heads]")
    a.lse_out = _dev(lse_out, torch.float32, "lse_out", optional=True)
    return a


def kvw_decode_attention(*, mode, q, k_cache, v_cache, context_lens, max_context, num_blocks,
                         block_size, out, block_table=None, num_blocks_per_req=None,
                         range_start=None, range_len=None, range_cum=None, num_ranges=None,
                         scale=None, workspace=None, err_flag=None, stream=None,
                         chunk_positions=0, cp_world_size=1, cp_rank=0, cp_interleave_size=1,
                         lse_out=None):
    """Decode attention over the paged cache (see include/kvw.h).

    q: [num_reqs, num_q_heads, head_dim] 2-byte (bf16) tensor; k_cache, v_cache:
    [num_blocks * block_size, num_kv_heads, head_dim]; out: float32 like q.  workspace:
    a byte tensor of kvw_decode_workspace_size(...) bytes, allocated here when None.
    """
    if workspace is None:
        need = kvw_decode_workspace_size(int(q.shape[0]), int(max_context), int(q.shape[1]),
                                         int(q.shape[2]))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    a = _decode_args(mode, q, k_cache, v_cache, context_lens, max_context, num_blocks, block_size,
                     out, block_table, num_blocks_per_req, range_start, range_len, range_cum,
                     num_ranges, scale, workspace, err_flag, chunk_positions, cp_world_size,
                     cp_rank, cp_interleave_size, lse_out)
    _check(library().kvw_decode_attention(ctypes.byref(a), _stream(stream)))


def kvw_decode_attention_noalloc(*, mode, q, k_cache, v_cache, context_lens, max_context,
                                 num_blocks, block_size, out, block_table=None,
                                 num_blocks_per_req=None, range_start=None, range_len=None,
                                 range_cum=None, num_ranges=None, scale=None, err_flag=None,
                                 stream=None, chunk_positions=0, cp_world_size=1, cp_rank=0,
                                 cp_interleave_size=1, lse_out=None):
    """kvw_decode_attention with the library's static per-GPU workspace (see include/kvw.h):
    nothing is allocated, here or in the library."""
    a = _decode_args(mode, q, k_cache, v_cache, context_lens, max_context, num_blocks, block_size,
                     out, block_table, num_blocks_per_req, range_start, range_len, range_cum,
                     num_ranges, scale, None, err_flag, chunk_positions, cp_world_size, cp_rank,
                     cp_interleave_size, lse_out)
    _check(library().kvw_decode_attention_noalloc(ctypes.byref(a), _stream(stream)))


def kvw_decode_merge(outs, lses, out, lse_out=None, stream=None):
    """Merge decode attention over disjoint position sets (see include/kvw.h).

    outs: float32 [parts, num_reqs, num_q_heads, head_dim]; lses: float32 [parts, num_reqs,
    num_q_heads]; out: float32 [num_reqs, num_q_heads, head_dim]; lse_out: optional float32
    [num_reqs, num_q_heads].
    """
    if outs.dim() != 4 or tuple(lses.shape) != tuple(outs.shape[:3]) or \
            tuple(out.shape) != tuple(outs.shape[1:]):
        raise ValueError("outs [P, R, Hq, D], lses [P, R, Hq] and out [R, Hq, D] must agree")
    parts, num_reqs, hq, d = (int(x) for x in outs.shape)
    _check(library().kvw_decode_merge(parts, num_reqs, hq, d,
                                      _dev(outs, torch.float32, "outs"),
                                      _dev(lses, torch.float32, "lses"),
                                      _dev(out, torch.float32, "out"),
                                      _dev(lse_out, torch.float32, "lse_out", optional=True),
                                      _stream(stream)))
