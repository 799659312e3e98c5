"""The C-ABI library on the CPU: it loads, exports what include/kvw.h declares, and its
host-side validation rejects bad arguments before anything is enqueued.

Every call below fails validation (or has no token rows), so no HIP call is made.
"""
import ctypes
import os
import re
import subprocess

import pytest

import paged_kv_cache_46_amd as kvw
from paged_kv_cache_46_amd.build import LIBRARY

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvw.h")
INCLUDE_DIR = os.path.join(ROOT, "include")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))
OK, INVALID, UNSUPPORTED, RANGE_CAP, HIP = range(5)
P = 0x10000  # an aligned, never dereferenced stand-in for a device pointer


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        # header-only helpers (static inline, with their bodies) are not library symbols
        text = re.sub(r"static inline[^{]*\{.*?\n\}", "", text, flags=re.S)
        names.update(re.findall(r"\b(kvw_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def inline_helpers():
    """Functions the headers define static inline."""
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"static inline\s+\w+\s+(kvw_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIBRARY):
        pytest.fail("libkvw.so is not built (run __graft_entry__.build())")
    return kvw.library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kvw_slot_mapping_paged", "kvw_slot_mapping_ranges",
                     "kvw_map_to_kernel_blocks", "kvw_ranges_to_block_table", "kvw_kv_write",
                     "kvw_alloc_create", "kvw_alloc_extend", "kvw_alloc_ranges",
                     "kvw_coord_offset"):
        assert required in names


def test_inline_offset_matches_the_library():
    """The header's inline offset, compiled into a small C program, against the exported
    kvw_coord_offset on in-range, out-of-range and overflowing coordinates (status and value)."""
    assert inline_helpers() == ["kvw_coord_offset_inline"]
    import tempfile
    src = r'''
#include <stdio.h>
#include "kvw_alloc.h"
int main(void) {
    const int64_t c[][7] = {
        {3, 100, 7, 32, 65536, 32, 2048}, {31, 65535, 31, 32, 65536, 32, 2048},
        {32, 0, 0, 32, 65536, 32, 2048}, {-1, 0, 0, 32, 65536, 32, 2048},
        {0, 0, 0, 1, 1, 1, -1}, {1, 5, 7, 2, 1LL << 40, 1LL << 40, 0},
        {0, 0, (1LL << 62) - 1, 1, 1, 1LL << 62, 2}, {0, 0, (1LL << 62) - 1, 1, 1, 1LL << 62, 3},
        {(1LL << 40) - 1, 1, 0, 1LL << 40, 1LL << 40, 1, 1LL << 30}};
    for (unsigned i = 0; i < sizeof c / sizeof c[0]; ++i) {
        int64_t a = -7, b = -7;
        const int sa = kvw_coord_offset_inline(c[i][0], c[i][1], c[i][2], c[i][3], c[i][4],
                                               c[i][5], c[i][6], &a);
        const int sb = kvw_coord_offset(c[i][0], c[i][1], c[i][2], c[i][3], c[i][4], c[i][5],
                                        c[i][6], &b);
        printf("%d %lld %d %lld\n", sa, (long long)a, sb, (long long)b);
    }
    return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c_file, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        with open(c_file, "w") as f:
            f.write(src)
        subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-I", INCLUDE_DIR, c_file,
                        "-L", os.path.dirname(LIBRARY), "-lkvw", "-Wl,-rpath," +
                        os.path.dirname(LIBRARY), "-Wl,-rpath-link,/opt/rocm/lib", "-o", exe],
                       check=True)
        rows = [ln.split() for ln in subprocess.run([exe], capture_output=True, text=True,
                                                    check=True).stdout.splitlines()]
    assert len(rows) == 9
    for sa, a, sb, b in rows:
        assert sa == sb and (a == b or sa != "0")
    assert [int(r[0]) for r in rows] == [0, 0, 1, 1, 1, 0, 0, 2, 2]
    assert int(rows[0][1]) == ((3 * 65536 + 100) * 32 + 7) * 2048
    assert int(rows[5][1]) == 0 and int(rows[6][1]) == 2 * ((1 << 62) - 1)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIBRARY], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (kvw_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version_and_struct_layout(lib):
    assert lib.kvw_abi_version() == kvw.kvw.KVW_ABI_VERSION
    assert lib.kvw_kv_write_args_size() == ctypes.sizeof(kvw.kvw.kvw_kv_write_args)
    text = open(HEADER).read()
    assert f"#define KVW_ABI_VERSION {kvw.kvw.KVW_ABI_VERSION}" in text
    fields = re.search(r"typedef struct kvw_kv_write_args \{(.*?)\} kvw_kv_write_args;", text, re.S)
    c_names = re.findall(r"\*?\s*(\w+);", re.sub(r"/\*.*?\*/", "", fields.group(1), flags=re.S))
    assert c_names == [f[0] for f in kvw.kvw.kvw_kv_write_args._fields_]
    assert lib.kvw_decode_args_size() == ctypes.sizeof(kvw.kvw.kvw_decode_args)
    fields = re.search(r"typedef struct kvw_decode_args \{(.*?)\} kvw_decode_args;", text, re.S)
    c_names = re.findall(r"\*?\s*(\w+);", re.sub(r"/\*.*?\*/", "", fields.group(1), flags=re.S))
    assert c_names == [f[0] for f in kvw.kvw.kvw_decode_args._fields_]


def _err(lib):
    return lib.kvw_last_error().decode()


def test_slot_mapping_validation(lib):
    f = lib.kvw_slot_mapping_paged
    NO_CP = (1, 0, 1)
    assert f(P, 4, P, 512, P, 16, P, 0, *NO_CP, P, None, None) == INVALID   # block_size 0
    assert "block_size" in _err(lib)
    assert f(P, 4, P, -1, P, 16, P, 16, *NO_CP, P, None, None) == INVALID   # negative token rows
    assert f(P, 4, P, 1 << 31, P, 16, P, 16, *NO_CP, P, None, None) == INVALID
    assert f(P, -1, P, 512, P, 16, P, 16, *NO_CP, P, None, None) == INVALID
    assert f(None, 4, P, 512, P, 16, P, 16, *NO_CP, P, None, None) == INVALID
    assert f(P, 4, P + 4, 512, P, 16, P, 16, *NO_CP, P, None, None) == INVALID  # misaligned int64
    assert f(P, 4, P, 512, None, 16, P, 16, *NO_CP, P, None, None) == INVALID   # table missing
    assert f(P, 4, P, 512, P, -2, P, 16, *NO_CP, P, None, None) == INVALID
    assert f(P, 4, P, 512, P, 16, P, 16, *NO_CP, None, None, None) == INVALID  # output missing
    assert f(P, 4, P, 512, P, 16, P, 16, *NO_CP, P, P + 2, None) == INVALID   # misaligned err_flag
    assert f(P, 4, P, 0, P, 16, P, 16, *NO_CP, None, None, None) == OK        # nothing to do
    g = lib.kvw_slot_mapping_ranges
    assert g(P, 4, P, 512, P, P, P, P, 65537, 16, *NO_CP, P, None, None) == RANGE_CAP
    assert g(P, 4, P, 512, None, P, P, P, 8, 16, *NO_CP, P, None, None) == INVALID
    assert g(P, 4, P, 512, P, P, P, P, -1, 16, *NO_CP, P, None, None) == INVALID


def test_context_parallel_validation(lib):
    f = lib.kvw_slot_mapping_paged
    for cp, what in (((-1, 0, 1), "negative"), ((2, 2, 1), "cp_rank"), ((2, -1, 1), "cp_rank"),
                     ((2, 0, 3), "divide"), ((2, 0, 0), "divide"), ((1, 1, 1), "cp_rank"),
                     ((1 << 28, 0, 1), "overflows")):
        assert f(P, 4, P, 512, P, 16, P, 16, *cp, P, None, None) == INVALID, cp
        assert what in _err(lib), (cp, _err(lib))
        assert lib.kvw_slot_mapping_ranges(P, 4, P, 512, P, P, P, P, 8, 16, *cp, P, None,
                                           None) == INVALID
    for cp in ((0, 5, 0), (1, 0, 1), (4, 3, 16), (8, 0, 2)):   # world 0: rank and interleave unused
        assert f(P, 4, P, 0, P, 16, P, 16, *cp, None, None, None) == OK, cp


def test_expansion_validation(lib):
    f = lib.kvw_map_to_kernel_blocks
    assert f(P, None, 2, 4, 32, 12, P, 16, None, None) == INVALID  # does not divide
    assert "does not divide" in _err(lib)
    assert f(P, None, 2, 4, 16, 32, P, 16, None, None) == INVALID
    assert f(P, None, 2, 4, 32, 0, P, 16, None, None) == INVALID
    assert f(P, None, 2, 4, 32, 16, P, 7, None, None) == INVALID   # out_stride < in_stride*k
    assert f(P, None, 0, 4, 32, 16, P, 8, None, None) == OK        # no rows
    g = lib.kvw_map_ranges_to_kernel_blocks
    assert g(P, P, P, P, 2, 4, 32, 12, P, P, P, P, None, None) == INVALID
    assert g(P, P, P, P, 2, 70000, 32, 16, P, P, P, P, None, None) == RANGE_CAP


def test_table_fill_validation(lib):
    f = lib.kvw_ranges_to_block_table
    # start, len, cum, num_ranges, rows, range_stride, bs, kernel bs, table, table stride,
    # counts, err_flag, stream
    assert f(P, P, P, P, 2, 4, 32, 12, P, 16, None, None, None) == INVALID  # does not divide
    assert "does not divide" in _err(lib)
    assert f(P, P, P, P, 2, 4, 32, 0, P, 16, None, None, None) == INVALID
    assert f(P, P, P, P, 2, 70000, 32, 16, P, 16, None, None, None) == RANGE_CAP
    assert f(P, P, P, None, 2, 4, 32, 16, P, 16, None, None, None) == INVALID  # num_ranges
    assert f(None, P, P, P, 2, 4, 32, 16, P, 16, None, None, None) == INVALID
    assert f(P, P, P + 2, P, 2, 4, 32, 16, P, 16, None, None, None) == INVALID  # misaligned cum
    assert f(P, P, P, P, 2, 4, 32, 16, None, 16, None, None, None) == INVALID  # table missing
    assert f(P, P, P, P, 2, 4, 32, 16, P, -1, None, None, None) == INVALID
    assert f(P, P, P, P, -1, 4, 32, 16, P, 16, None, None, None) == INVALID
    assert f(P, P, P, P, 2, 4, 32, 16, P, 16, P + 1, None, None) == INVALID  # counts misaligned
    assert f(P, P, P, P, 2, 4, 32, 16, P, 16, None, P + 3, None) == INVALID  # err_flag misaligned
    assert f(P, P, P, P, 0, 4, 32, 16, P, 16, None, None, None) == OK        # no rows


def _args(**kw):
    a = kvw.kvw.kvw_kv_write_args()
    base = dict(mode=kvw.KVW_SLOTS_PAGED, num_reqs=4, query_start_loc=P, positions=P,
                max_num_tokens=512, block_table=P, block_table_stride=16, block_size=16,
                num_layers=1, num_blocks=512, key=P, value=P, kv_layer_stride=0,
                kv_token_stride=2048, k_cache=P, v_cache=P, bytes_per_token=2048,
                slot_mapping_in=P, range_start=P, range_len=P, range_cum=P, num_ranges=P,
                range_stride=4)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


def test_kv_write_validation(lib):
    f = lib.kvw_kv_write
    assert f(None, None) == INVALID
    assert f(ctypes.byref(_args(mode=7)), None) == INVALID
    assert f(ctypes.byref(_args(bytes_per_token=24)), None) == INVALID
    assert f(ctypes.byref(_args(bytes_per_token=0)), None) == INVALID
    assert f(ctypes.byref(_args(bytes_per_token=1 << 31)), None) == INVALID  # a row below 2 GiB
    assert f(ctypes.byref(_args(key=P + 8)), None) == INVALID
    assert f(ctypes.byref(_args(kv_token_stride=2056)), None) == INVALID
    assert f(ctypes.byref(_args(k_cache=None)), None) == INVALID
    assert f(ctypes.byref(_args(num_blocks=1 << 62)), None) == INVALID  # cache size overflow
    assert f(ctypes.byref(_args(block_size=-16)), None) == INVALID
    assert f(ctypes.byref(_args(mode=kvw.KVW_SLOTS_RANGES, range_stride=1 << 20)), None) == RANGE_CAP
    assert f(ctypes.byref(_args(mode=kvw.KVW_SLOTS_PRECOMPUTED, slot_mapping_in=None)), None) == INVALID
    assert f(ctypes.byref(_args(schedule=3)), None) == INVALID
    assert "schedule" in _err(lib)
    assert f(ctypes.byref(_args(schedule=kvw.KVW_SCHEDULE_TWO_KERNELS, slot_mapping_out=None)),
             None) == INVALID
    assert f(ctypes.byref(_args(cp_world_size=2, cp_rank=2)), None) == INVALID
    assert f(ctypes.byref(_args(cp_world_size=2, cp_interleave_size=5)), None) == INVALID
    assert f(ctypes.byref(_args(table_out=P, table_out_stride=32, table_block_size=5)),
             None) == INVALID                                   # does not divide block_size
    assert f(ctypes.byref(_args(table_out=P, table_out_stride=31, table_block_size=8)),
             None) == INVALID                                   # below block_table_stride * k
    assert f(ctypes.byref(_args(table_out=P, table_out_stride=0, table_block_size=8)),
             None) == INVALID
    assert f(ctypes.byref(_args(table_out=P + 2, table_out_stride=32, table_block_size=8)),
             None) == INVALID                                   # misaligned
    assert f(ctypes.byref(_args(mode=kvw.KVW_SLOTS_PRECOMPUTED, table_out=P, table_out_stride=32,
                                table_block_size=8)), None) == INVALID
    assert f(ctypes.byref(_args(max_num_tokens=0)), None) == OK


def test_binding_rejects_missing_library(tmp_path):
    from paged_kv_cache_46_amd import kvw as binding
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            binding.library(str(tmp_path / "absent.so"))
    finally:
        binding._lib = saved


def _decode(**kw):
    a = kvw.kvw.kvw_decode_args()
    base = dict(mode=kvw.KVW_SLOTS_PAGED, num_reqs=4, q=P, context_lens=P, max_context=1000,
                block_size=16, block_table=P, num_blocks_per_req=P, block_table_stride=64,
                range_stride=8, range_start=P, range_len=P, range_cum=P, num_ranges=P,
                k_cache=P, v_cache=P, num_blocks=256, num_q_heads=32, num_kv_heads=8,
                head_dim=128, scale=0.088, out=P, workspace=P, workspace_bytes=1 << 30)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


def test_decode_workspace_size(lib):
    ws = lib.kvw_decode_workspace_size
    ws.restype = ctypes.c_int64
    # per request and 256 positions: per query head 128 sums, the chunk max and sum (fp32), and
    # one 8-byte work-list entry; then 16 bytes for the list's length
    assert ws(4, 1000, 32, 128) == 4 * 4 * (32 * 130 * 4 + 8) + 16
    assert ws(4, 1024, 32, 128) == 4 * 4 * (32 * 130 * 4 + 8) + 16
    assert ws(4, 1025, 32, 128) == 4 * 5 * (32 * 130 * 4 + 8) + 16
    assert ws(4, 0, 32, 128) == 16
    assert ws(-1, 10, 32, 128) == -1
    # sizes whose product does not fit int64 (head_dim + 2 itself past int32 here)
    assert ws(65535, 2**31 - 1, 2**31 - 1, 2**31 - 1) == -1
    assert ws(1, 256, 1, 2**31 - 1) == (2**31 + 1) * 4 + 8 + 16


def test_decode_validation(lib):
    f = lib.kvw_decode_attention
    assert f(None, None) == INVALID
    assert f(ctypes.byref(_decode(mode=kvw.KVW_SLOTS_PRECOMPUTED)), None) == INVALID
    assert f(ctypes.byref(_decode(head_dim=64)), None) == UNSUPPORTED
    assert f(ctypes.byref(_decode(num_q_heads=128, num_kv_heads=16)), None) == UNSUPPORTED  # G=8, 16 kv
    assert f(ctypes.byref(_decode(num_q_heads=12, num_kv_heads=4)), None) == UNSUPPORTED  # 3 per head
    assert f(ctypes.byref(_decode(num_q_heads=32, num_kv_heads=32)), None) == UNSUPPORTED  # 32 kv heads
    assert f(ctypes.byref(_decode(num_q_heads=16, num_kv_heads=1)), None) == UNSUPPORTED  # 16 per head
    assert f(ctypes.byref(_decode(num_q_heads=30, num_kv_heads=8)), None) == UNSUPPORTED
    assert f(ctypes.byref(_decode(block_size=0)), None) == INVALID
    assert f(ctypes.byref(_decode(max_context=-1)), None) == INVALID
    assert f(ctypes.byref(_decode(num_reqs=70000)), None) == INVALID
    assert f(ctypes.byref(_decode(num_blocks=1 << 60)), None) == INVALID   # cache size overflow
    assert f(ctypes.byref(_decode(q=P + 4)), None) == INVALID
    assert f(ctypes.byref(_decode(out=None)), None) == INVALID
    assert f(ctypes.byref(_decode(k_cache=P + 8)), None) == INVALID
    assert f(ctypes.byref(_decode(err_flag=P + 2)), None) == INVALID
    assert f(ctypes.byref(_decode(block_table=None)), None) == INVALID
    assert f(ctypes.byref(_decode(block_table_stride=-1)), None) == INVALID
    assert f(ctypes.byref(_decode(mode=kvw.KVW_SLOTS_RANGES, range_cum=None)), None) == INVALID
    assert f(ctypes.byref(_decode(mode=kvw.KVW_SLOTS_RANGES, range_stride=1 << 20)),
             None) == RANGE_CAP
    assert f(ctypes.byref(_decode(workspace_bytes=4 * 4 * (32 * 130 * 4 + 8) + 15)), None) == INVALID
    assert "workspace" in _err(lib)
    assert f(ctypes.byref(_decode(workspace=None)), None) == INVALID
    assert f(ctypes.byref(_decode(chunk_positions=128)), None) == INVALID
    assert f(ctypes.byref(_decode(chunk_positions=768)), None) == INVALID
    assert f(ctypes.byref(_decode(chunk_positions=4096)), None) == INVALID
    assert f(ctypes.byref(_decode(cp_world_size=2, cp_rank=2, cp_interleave_size=1)), None) == INVALID
    assert f(ctypes.byref(_decode(cp_world_size=2, cp_rank=1, cp_interleave_size=3)), None) == INVALID
    assert f(ctypes.byref(_decode(cp_world_size=-1)), None) == INVALID
    assert f(ctypes.byref(_decode(lse_out=P + 2)), None) == INVALID
    assert f(ctypes.byref(_decode(num_reqs=0)), None) == OK   # nothing to do: no launch


def test_decode_noalloc_validation(lib):
    """The static-workspace variant validates like kvw_decode_attention (its workspace
    arguments are ignored) and rejects, before any HIP call, sizes whose workspace exceeds
    the static array."""
    f = lib.kvw_decode_attention_noalloc
    assert f(None, None) == INVALID
    assert f(ctypes.byref(_decode(mode=kvw.KVW_SLOTS_PRECOMPUTED)), None) == INVALID
    assert f(ctypes.byref(_decode(head_dim=64)), None) == UNSUPPORTED
    assert f(ctypes.byref(_decode(block_size=0)), None) == INVALID
    assert f(ctypes.byref(_decode(q=P + 4)), None) == INVALID
    assert f(ctypes.byref(_decode(mode=kvw.KVW_SLOTS_RANGES, range_stride=1 << 20)),
             None) == RANGE_CAP
    assert f(ctypes.byref(_decode(chunk_positions=768)), None) == INVALID
    assert f(ctypes.byref(_decode(num_reqs=0, workspace=None, workspace_bytes=0)), None) == OK
    # 64 requests of 131,072 positions, 32 query heads: the library's chunk for 32 requests or
    # more is 1024, so 64 * 128 chunks of 32 * 130 fp32 partials (136 MB) plus the work list
    big = _decode(num_reqs=64, max_context=131072, workspace=None, workspace_bytes=0)
    assert f(ctypes.byref(big), None) == UNSUPPORTED
    need = 64 * 128 * 32 * 130 * 4 + 64 * 128 * 8 + 4
    assert f"{need} bytes" in _err(lib) and str(64 << 20) in _err(lib)
    # at 2048-position chunks the same batch still needs 68 MB
    big2 = _decode(num_reqs=64, max_context=131072, chunk_positions=2048, workspace=None,
                   workspace_bytes=0)
    assert f(ctypes.byref(big2), None) == UNSUPPORTED


def test_decode_merge_validation(lib):
    f = lib.kvw_decode_merge
    assert f(0, 4, 32, 128, P, P, P, None, None) == INVALID        # no part
    assert f(2, 4, 32, 0, P, P, P, None, None) == INVALID          # head_dim
    assert f(2, 4, 32, 2048, P, P, P, None, None) == INVALID
    assert f(2, -1, 32, 128, P, P, P, None, None) == INVALID
    assert f(2, 4, 32, 128, None, P, P, None, None) == INVALID
    assert f(2, 4, 32, 128, P, P + 2, P, None, None) == INVALID
    assert f(2, 4, 32, 128, P, P, P, P + 1, None) == INVALID
    assert f(2, 0, 32, 128, P, P, P, None, None) == OK             # nothing to do: no launch
