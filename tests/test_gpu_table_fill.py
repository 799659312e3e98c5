"""Block table filled straight from range descriptors: HIP path vs CPU oracle (needs an MI355X).

Every table entry, every per-row count and the sticky flag word must equal
the oracle's exactly.  Outputs are pre-filled with -5 so that an entry the
kernel leaves unwritten shows up.  The manager block size is 16*k and the
kernel block size 16, so k is the expansion factor.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_46_amd as kvw
from parity import DEV, DeviceInputs, dev, host, new_flag, say
from workloads import config, long_context, range_tables, small_cases

pytestmark = pytest.mark.gpu

SMALL = small_cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvw.library()
    yield
    torch.cuda.synchronize()


def fill_and_compare(rs, rl, rc, nr, k, width, tag, with_counts=True):
    """Run the fill on the GPU and compare table, counts and flags with the oracle."""
    rows = rs.shape[0]
    say(f"[fill] {tag}: rows {rows} range_stride {rs.shape[1]} k {k} width {width}")
    o_t, o_c, o_f = oracle.get().ranges_to_block_table(rs, rl, rc, nr, 16 * k, 16, width)
    table = torch.full((rows, width), -5, dtype=torch.int32, device=DEV)
    counts = torch.full((rows,), -5, dtype=torch.int32, device=DEV) if with_counts else None
    flag = new_flag()
    kvw.kvw_ranges_to_block_table(dev(rs), dev(rl), dev(rc), dev(nr), 16 * k, 16, table, counts,
                                  flag)
    torch.cuda.synchronize()
    g_t = host(table)
    bad = np.argwhere(g_t != o_t)
    assert len(bad) == 0, f"{len(bad)} entries differ, first at {bad[:4].tolist()}"
    if with_counts:
        assert np.array_equal(host(counts), o_c)
    assert int(flag.item()) == o_f
    return o_t, o_c, o_f


@pytest.mark.parametrize("k", [1, 2])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_fill_small(w, k):
    exact = w.table_stride * k
    for width in (exact, exact + 37, max(1, exact // 2)):
        fill_and_compare(w.range_start, w.range_len, w.range_cum, w.num_ranges, k, width,
                         f"{w.name} width {width}")


@pytest.mark.parametrize("name", ["tiny_prefill", "decode_step", "mixed_chunked", "full_32_layer"])
def test_fill_study(name):
    w = config(name)
    o_t, o_c, o_f = fill_and_compare(w.range_start, w.range_len, w.range_cum, w.num_ranges, 1,
                                     w.table_stride, name)
    # at k = 1 the filled table is the workload's own table
    assert o_f == 0 and np.array_equal(o_t, w.block_table)


@pytest.mark.parametrize("r", [1, 16, 512, 4096])
def test_fill_long_context(r):
    """128K context, manager runs (bs 32) -> kernel table (bs 16); slots through it match."""
    w = long_context(r)
    k = w.blocks_per_kv_block
    d = DeviceInputs(w)
    width = w.table_stride * k
    say(f"[fill] {w.describe()}")
    table = torch.full((w.max_num_reqs, width), -5, dtype=torch.int32, device=DEV)
    counts = torch.full((w.max_num_reqs,), -5, dtype=torch.int32, device=DEV)
    flag = new_flag()
    kvw.kvw_ranges_to_block_table(d.rs, d.rl, d.rc, d.nr, w.block_size, w.kernel_block_size,
                                  table, counts, flag)
    orc = oracle.get()
    o_t, o_c, o_f = orc.ranges_to_block_table(w.range_start, w.range_len, w.range_cum,
                                              w.num_ranges, w.block_size, w.kernel_block_size,
                                              width)
    torch.cuda.synchronize()
    assert np.array_equal(host(table), o_t) and np.array_equal(host(counts), o_c)
    assert int(flag.item()) == o_f == 0
    sm = torch.empty(w.max_num_tokens, dtype=torch.int64, device=DEV)
    kvw.kvw_slot_mapping_paged(d.qsl, w.num_reqs, d.positions, w.max_num_tokens, table, counts,
                               w.kernel_block_size, sm, flag)
    o_slots, _ = orc.slot_mapping_ranges(w.query_start_loc, w.num_reqs, w.positions,
                                         w.max_num_tokens, w.range_start, w.range_len,
                                         w.range_cum, w.num_ranges, w.block_size)
    torch.cuda.synchronize()
    assert np.array_equal(host(sm), o_slots) and int(flag.item()) == 0


@pytest.mark.parametrize("case", ["long_rows", "window_edges", "single_blocks"])
def test_fill_descriptor_shapes(case):
    """Rows with many runs: beyond one 128-entry search window, at its edges, and len-1 runs."""
    if case == "long_rows":
        runs, max_len, k = [20000, 129, 0, 65536, 3], 3, 2
    elif case == "window_edges":
        runs, max_len, k = [127, 128, 129, 255, 256, 257, 4095, 4096, 4097], 2, 1
    else:
        runs, max_len, k = [4096, 4096, 64, 65], 1, 4
    rs, rl, rc, nr = range_tables(4900 + len(case), runs, max_len=max_len)
    total = int((rl.sum(axis=1) * k).max())
    for width in (total, total + 300, total // 3 + 1):
        fill_and_compare(rs, rl, rc, nr, k, width, f"{case} width {width}")


def test_fill_many_rows():
    """More rows than one launch dimension holds: rows past 65,535 are looped over."""
    rng = np.random.default_rng(4950)
    runs = rng.integers(0, 3, size=70003).tolist()
    rs, rl, rc, nr = range_tables(4950, runs, max_len=2, range_stride=2)
    fill_and_compare(rs, rl, rc, nr, 2, 5, "many rows")


def test_fill_flags():
    """Clamped counts, truncated rows and ids that cannot be stored are flagged as the oracle says."""
    rs, rl, rc, nr = range_tables(4960, [6, 6, 3, 2, 4], max_len=3, range_stride=6)
    nr[1] = 9                     # above the stride: clamped to 6
    nr[3] = -2                    # negative: clamped to 0
    rs[0, 2] = -10                # negative block
    rs[2, 1] = (1 << 30) - 1      # at k = 2 the first kernel id pair fits, the next block's does not
    rl[2, 1] = 2
    rl[2, 2] = 1
    rc[2, 2] = rc[2, 1] + 2
    for width in (40, 7, 1):
        _, _, f = fill_and_compare(rs, rl, rc, nr, 2, width, f"flags width {width}")
        assert f & kvw.KVW_FLAG_COUNT
    _, _, f = fill_and_compare(rs, rl, rc, nr, 2, 40, "flags, no counts", with_counts=False)
    assert f == kvw.KVW_FLAG_COUNT | kvw.KVW_FLAG_BAD_BLOCK


def test_fill_empty():
    rs, rl, rc, nr = range_tables(4970, [2, 0, 3], max_len=2)
    fill_and_compare(rs, rl, rc, nr, 1, 0, "zero width")      # counts only: all clamped to 0
    e = np.zeros((0, 4), np.int32)
    fill_and_compare(e, e, e, np.zeros(0, np.int32), 2, 8, "zero rows")
    z = np.zeros((3, 0), np.int32)
    fill_and_compare(z, z, z, np.zeros(3, np.int32), 2, 8, "zero range stride")
