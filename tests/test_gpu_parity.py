"""HIP path vs CPU oracle, element by element, through the C-ABI (needs an MI355X).

Slot ids are compared exactly; cache planes are compared byte for byte
(the write is a copy: tolerance 0); the sticky flag word must equal the
oracle's flag bits.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_46_amd as kvw
from parity import (DEV, Caches, DeviceInputs, compare_caches, dev, gpu_slots, host, kv_device,
                    new_flag, oracle_slots, say)
import oracle
from workloads import BF16_SENTINEL, config, custom, long_context, small_cases
from workloads.gen import Request

pytestmark = pytest.mark.gpu

SMALL = small_cases()
MODES = {"precomputed": kvw.KVW_SLOTS_PRECOMPUTED, "paged": kvw.KVW_SLOTS_PAGED,
         "ranges": kvw.KVW_SLOTS_RANGES}
# fused modes: automatic schedule, forced two-kernel and one-kernel schedules (slot mapping
# kept), and no slot-mapping output (always one kernel)
WRITE_MODES = ["precomputed", "paged", "ranges", "paged-two", "ranges-two", "paged-one",
               "ranges-one", "paged-noslots", "ranges-noslots"]
SCHEDULES = {"": kvw.KVW_SCHEDULE_AUTO, "two": kvw.KVW_SCHEDULE_TWO_KERNELS,
             "one": kvw.KVW_SCHEDULE_ONE_KERNEL, "noslots": kvw.KVW_SCHEDULE_AUTO}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvw.library()
    yield
    torch.cuda.synchronize()


def run_kv_write(w, d, mode, caches, key, value, slots_in=None, block_size=None, num_blocks=None,
                 over=None):
    """Returns (slot_mapping_out or None, flags)."""
    over = over or {}
    mode, _, sched = mode.partition("-")
    keep = sched != "noslots"
    flag = new_flag()
    sm_out = torch.full((w.max_num_tokens,), 777, dtype=torch.int64, device=DEV)
    kw = dict(mode=MODES[mode], key=key, value=value, k_cache=caches.k, v_cache=caches.v,
              num_blocks=num_blocks or w.num_blocks, block_size=block_size or w.block_size,
              max_num_tokens=w.max_num_tokens, err_flag=flag, schedule=SCHEDULES[sched])
    if mode == "precomputed":
        kw["slot_mapping_in"] = dev(slots_in)
    else:
        kw.update(query_start_loc=d.qsl, num_reqs=w.num_reqs, positions=d.positions,
                  slot_mapping_out=sm_out if keep else None)
        if mode == "paged":
            kw.update(block_table=over.get("block_table", d.block_table),
                      num_blocks_per_req=over.get("nbpr", d.nbpr))
        else:
            kw.update(range_start=over.get("rs", d.rs), range_len=over.get("rl", d.rl),
                      range_cum=over.get("rc", d.rc), num_ranges=over.get("nr", d.nr))
    kvw.kvw_kv_write(**kw)
    torch.cuda.synchronize()
    return (host(sm_out) if keep else None), int(flag.item())


def check_kv_write(w, mode, **over):
    say(f"[kv_write] {w.describe()} mode={mode}")
    d = DeviceInputs(w)
    variant = "ranges" if mode.startswith("ranges") else "paged"
    o_slots, o_flags = oracle_slots(w, variant)
    key_h, value_h = w.kv_plane(0), w.kv_plane(1)
    key = dev(key_h).view(w.num_layers, w.max_num_tokens, w.num_kv_heads, w.head_dim)
    value = dev(value_h).view_as(key)
    caches = Caches(w.num_layers, w.num_blocks, w.block_size, w.row_elems)
    sm, flags = run_kv_write(w, d, mode, caches, key, value, slots_in=o_slots)
    if mode == "precomputed":
        o_flags = 0
    elif sm is not None:
        assert np.array_equal(sm, o_slots), f"{w.name}: fused slot_mapping_out differs"
    c_flags = compare_caches(w, caches, o_slots, key_h, value_h, w.num_blocks, w.block_size)
    assert flags == o_flags | c_flags


# ---------------------------------------------------------------------------
# slot mapping
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", ["paged", "ranges"])
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_slot_mapping_small(w, variant):
    say(f"[slots] {w.describe()} {variant}")
    g, gf = gpu_slots(w, DeviceInputs(w), variant)
    o, of = oracle_slots(w, variant)
    assert np.array_equal(g, o)
    assert gf == of


STUDY = ["tiny_prefill", "decode_step", "mixed_chunked", "full_32_layer"]


@pytest.mark.parametrize("variant", ["paged", "ranges"])
@pytest.mark.parametrize("name", STUDY)
def test_slot_mapping_study(name, variant):
    w = config(name)
    say(f"[slots] {w.describe()} {variant}")
    g, gf = gpu_slots(w, DeviceInputs(w), variant)
    o, of = oracle_slots(w, variant)
    assert np.array_equal(g, o) and gf == of == 0


@pytest.mark.parametrize("r", [1, 16, 512, 4096])
def test_long_context_slots_and_expansion(r):
    """128K context: expansion 32->16 on the GPU, then both variants, against the oracle chain."""
    w = long_context(r)
    say(f"[expand+slots] {w.describe()}")
    orc = oracle.get()
    d = DeviceInputs(w)
    k = w.blocks_per_kv_block
    # block-table expansion
    kt = torch.full((w.max_num_reqs, w.table_stride * k), -5, dtype=torch.int32, device=DEV)
    flag = new_flag()
    kvw.kvw_map_to_kernel_blocks(d.block_table, d.nbpr, w.block_size, w.kernel_block_size, kt, flag)
    o_kt, of = orc.map_to_kernel_blocks(w.block_table, w.num_blocks_per_req, w.block_size,
                                        w.kernel_block_size)
    torch.cuda.synchronize()
    assert np.array_equal(host(kt), o_kt) and int(flag.item()) == of == 0
    # range expansion
    outs = [torch.full_like(d.rs, -5) for _ in range(3)] + [torch.full_like(d.nr, -5)]
    kvw.kvw_map_ranges_to_kernel_blocks(d.rs, d.rl, d.rc, d.nr, w.block_size, w.kernel_block_size,
                                        *outs, err_flag=flag)
    (o_s, o_l, o_c, o_n), of = orc.map_ranges_to_kernel_blocks(
        w.range_start, w.range_len, w.range_cum, w.num_ranges, w.block_size, w.kernel_block_size)
    torch.cuda.synchronize()
    for g_, o_ in zip(outs, (o_s, o_l, o_c, o_n)):
        assert np.array_equal(host(g_), o_)
    # slot mapping at kernel block size through the GPU-expanded table and ranges
    nb_k = d.nbpr * k
    sm = torch.empty(w.max_num_tokens, dtype=torch.int64, device=DEV)
    kvw.kvw_slot_mapping_paged(d.qsl, w.num_reqs, d.positions, w.max_num_tokens, kt, nb_k,
                               w.kernel_block_size, sm, flag)
    o_paged, _ = orc.slot_mapping_paged(w.query_start_loc, w.num_reqs, w.positions,
                                        w.max_num_tokens, o_kt, w.num_blocks_per_req * k,
                                        w.kernel_block_size)
    torch.cuda.synchronize()
    assert np.array_equal(host(sm), o_paged)
    kvw.kvw_slot_mapping_ranges(d.qsl, w.num_reqs, d.positions, w.max_num_tokens, *outs,
                                w.kernel_block_size, sm, flag)
    torch.cuda.synchronize()
    assert np.array_equal(host(sm), o_paged)
    # and the manager-unit ranges at block size 32 give the same slots
    kvw.kvw_slot_mapping_ranges(d.qsl, w.num_reqs, d.positions, w.max_num_tokens, d.rs, d.rl,
                                d.rc, d.nr, w.block_size, sm, flag)
    torch.cuda.synchronize()
    assert np.array_equal(host(sm), o_paged)
    assert int(flag.item()) == 0


# ---------------------------------------------------------------------------
# K/V write with the attention-side table made in the same launch
# ---------------------------------------------------------------------------
def check_kv_write_with_table(w, mode, k, pad=3, payload=None):
    """Fused write that also returns the kernel-unit block table: slots, caches, table, counts.
    payload: ((key_h, value_h), (key, value)) to use instead of the workload's own."""
    say(f"[kv_write+table] {w.describe()} mode={mode} k={k}")
    variant, _, sched = mode.partition("-")
    orc = oracle.get()
    d = DeviceInputs(w)
    o_slots, o_flags = oracle_slots(w, variant)
    kbs = w.block_size // k
    width = w.table_stride * k + pad
    if variant == "paged":
        o_table, o_counts, t_flags = orc.map_to_kernel_blocks(
            w.block_table, w.num_blocks_per_req, w.block_size, kbs, width, with_counts=True)
    else:
        o_table, o_counts, t_flags = orc.ranges_to_block_table(
            w.range_start, w.range_len, w.range_cum, w.num_ranges, w.block_size, kbs, width)
    if payload is None:
        key_h, value_h = w.kv_plane(0), w.kv_plane(1)
        key = dev(key_h).view(w.num_layers, w.max_num_tokens, w.num_kv_heads, w.head_dim)
        value = dev(value_h).view_as(key)
    else:
        (key_h, value_h), (key, value) = payload
    caches = Caches(w.num_layers, w.num_blocks, w.block_size, w.row_elems)
    table = torch.full((w.num_reqs, width), -5, dtype=torch.int32, device=DEV)
    counts = torch.full((w.num_reqs,), -5, dtype=torch.int32, device=DEV)
    flag = new_flag()
    sm = torch.full((w.max_num_tokens,), 777, dtype=torch.int64, device=DEV)
    kw = dict(query_start_loc=d.qsl, num_reqs=w.num_reqs, positions=d.positions,
              slot_mapping_out=None if sched == "noslots" else sm)
    if variant == "paged":
        kw.update(mode=kvw.KVW_SLOTS_PAGED, block_table=d.block_table, num_blocks_per_req=d.nbpr)
    else:
        kw.update(mode=kvw.KVW_SLOTS_RANGES, range_start=d.rs, range_len=d.rl, range_cum=d.rc,
                  num_ranges=d.nr)
    kvw.kvw_kv_write(key=key, value=value, k_cache=caches.k, v_cache=caches.v,
                     num_blocks=w.num_blocks, block_size=w.block_size,
                     max_num_tokens=w.max_num_tokens, err_flag=flag, schedule=SCHEDULES[sched],
                     table_out=table, table_counts_out=counts, table_block_size=kbs, **kw)
    torch.cuda.synchronize()
    bad = np.argwhere(host(table) != o_table)
    assert len(bad) == 0, f"{len(bad)} table entries differ, first {bad[:4].tolist()}"
    assert np.array_equal(host(counts), o_counts)
    if sched != "noslots":
        assert np.array_equal(host(sm), o_slots)
    c_flags = compare_caches(w, caches, o_slots, key_h, value_h, w.num_blocks, w.block_size)
    assert int(flag.item()) == o_flags | t_flags | c_flags


TABLE_MODES = ["paged", "ranges", "paged-two", "ranges-two", "paged-one", "ranges-one",
               "paged-noslots", "ranges-noslots"]


@pytest.mark.parametrize("mode", TABLE_MODES)
@pytest.mark.parametrize("w", [w for w in SMALL if w.name in (
    "tiny_prefill", "small_mixed_l3", "small_bs8", "small_bs64", "small_oversub", "small_dummy",
    "small_out_of_range", "small_empty")], ids=lambda w: w.name)
def test_kv_write_with_table(w, mode):
    check_kv_write_with_table(w, mode, k=2 if w.block_size % 2 == 0 else 1)


@pytest.mark.parametrize("mode", ["paged", "ranges", "paged-noslots", "ranges-noslots"])
@pytest.mark.parametrize("r", [1, 16, 512, 4096])
def test_kv_write_with_table_long_context(r, mode):
    """128K: the step's kernel-unit table (32 -> 16) written by the slot-mapping launch (or, in
    the one-kernel schedule, by a launch before it); slots, table, counts and the whole cache."""
    check_kv_write_with_table(long_context(r), mode, k=2, pad=0, payload=long_context_payload())


@pytest.mark.parametrize("mode", ["paged-two", "ranges-two", "paged-one", "ranges-one"])
def test_kv_write_with_table_flagged(mode):
    check_kv_write_with_table(_flagged_workload(), mode, k=2)


def test_kv_write_table_without_token_rows():
    """max_num_tokens == 0: nothing is copied, the table is still written."""
    w = config("tiny_prefill")
    d = DeviceInputs(w)
    orc = oracle.get()
    key = torch.zeros((1, 0, w.num_kv_heads, w.head_dim), dtype=torch.int16, device=DEV)
    caches = Caches(1, 4, w.block_size, w.row_elems)
    for variant in ("paged", "ranges"):
        table = torch.full((w.num_reqs, w.table_stride * 2), -5, dtype=torch.int32, device=DEV)
        counts = torch.full((w.num_reqs,), -5, dtype=torch.int32, device=DEV)
        mapping = (dict(mode=kvw.KVW_SLOTS_PAGED, block_table=d.block_table,
                        num_blocks_per_req=d.nbpr) if variant == "paged" else
                   dict(mode=kvw.KVW_SLOTS_RANGES, range_start=d.rs, range_len=d.rl,
                        range_cum=d.rc, num_ranges=d.nr))
        kvw.kvw_kv_write(key=key, value=key, k_cache=caches.k, v_cache=caches.v, num_blocks=4,
                         block_size=w.block_size, max_num_tokens=0, query_start_loc=d.qsl,
                         num_reqs=w.num_reqs, positions=d.positions, table_out=table,
                         table_counts_out=counts, table_block_size=w.block_size // 2, **mapping)
        torch.cuda.synchronize()
        if variant == "paged":
            o_t, o_c, _ = orc.map_to_kernel_blocks(w.block_table, w.num_blocks_per_req,
                                                   w.block_size, w.block_size // 2,
                                                   with_counts=True)
        else:
            o_t, o_c, _ = orc.ranges_to_block_table(w.range_start, w.range_len, w.range_cum,
                                                    w.num_ranges, w.block_size,
                                                    w.block_size // 2, w.table_stride * 2)
        assert np.array_equal(host(table), o_t) and np.array_equal(host(counts), o_c)
    assert (host(caches.t) == 0x7FC0).all()


# ---------------------------------------------------------------------------
# K/V write
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", WRITE_MODES)
@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_kv_write_small(w, mode):
    check_kv_write(w, mode)


def _row_width_workload(heads, head_dim):
    r = np.random.default_rng(4730 + heads * 131 + head_dim)
    reqs = [Request(int(r.integers(1, 3000)) + 700, int(r.integers(300, 700))) for _ in range(5)]
    reqs += [Request(int(r.integers(1, 3000)), 1) for _ in range(40)]
    n = sum(q.n_new for q in reqs)
    return custom(f"rows_{heads * head_dim * 2}B", 4730 + heads, reqs, block_size=16,
                  num_blocks=9000, runs=("count", 1, 5), num_kv_heads=heads, head_dim=head_dim,
                  num_layers=2, max_num_tokens=n + 29)


# rows of 48 B (21 tokens per wave), 512 B (2 per wave), 1008 B (one per wave, 63 lanes),
# 1040 B (just over one slice), 2048 B: the packed and the slice-granular scatter
ROW_WIDTHS = [(1, 24), (2, 128), (63, 8), (65, 8), (8, 128)]


@pytest.mark.parametrize("mode", ["precomputed", "paged-two", "ranges-two", "paged-one",
                                  "paged-noslots"])
@pytest.mark.parametrize("shape", ROW_WIDTHS, ids=lambda s: f"{s[0] * s[1] * 2}B")
def test_kv_write_row_widths(shape, mode):
    check_kv_write(_row_width_workload(*shape), mode)


def _wide_row_workload(heads, head_dim, layers):
    r = np.random.default_rng(4760 + heads * 131 + head_dim + layers)
    reqs = [Request(int(r.integers(1, 600)) + 700, int(r.integers(300, 700))) for _ in range(6)]
    reqs += [Request(int(r.integers(1, 1200)), 1) for _ in range(24)]
    n = sum(q.n_new for q in reqs)
    return custom(f"wide_{heads * head_dim * 2}B_L{layers}", 4760 + heads, reqs, block_size=16,
                  num_blocks=3000, runs=("count", 1, 5), num_kv_heads=heads, head_dim=head_dim,
                  num_layers=layers, max_num_tokens=n + 29)


# rows over 2 KiB: 2,064 B (a partial third slice), 3 KiB and 4 KiB (three and four slices per
# lane in the one-kernel write), 6 KiB (copied in two segments); one layer keeps the one-kernel
# write at one wave per token, four layers (over 8,192 token rows) at one wave per plane
WIDE_ROWS = [(129, 8), (12, 128), (16, 128), (24, 128)]


@pytest.mark.parametrize("layers", [1, 4])
@pytest.mark.parametrize("mode", ["precomputed", "paged-two", "paged-one", "ranges-one"])
@pytest.mark.parametrize("shape", WIDE_ROWS, ids=lambda s: f"{s[0] * s[1] * 2}B")
def test_kv_write_wide_rows(shape, mode, layers):
    check_kv_write(_wide_row_workload(*shape, layers), mode)


@pytest.mark.parametrize("mode", WRITE_MODES[1:])
@pytest.mark.parametrize("name", ["tiny_prefill", "decode_step", "mixed_chunked"])
def test_kv_write_study(name, mode):
    check_kv_write(config(name), mode)


def _short_prefills():
    """Many short prefill chunks over rows of one- and two-block runs: a wave of 64 tokens holds
    several requests, most positions lie below their request's last run, and the lanes outside
    the wave's first request search their own rows."""
    r = np.random.default_rng(4741)
    reqs = [Request(int(r.integers(40, 3000)), int(r.integers(1, 48))) for _ in range(70)]
    return custom("short_prefills", 4741, reqs, block_size=16, num_blocks=20000,
                  runs=("len", 1, 2), num_kv_heads=2, head_dim=64,
                  max_num_tokens=sum(q.n_new for q in reqs) + 37)


def _many_runs():
    """Rows of up to 41,000 one-block runs at block size 1 (range_stride 41,000): finding a run
    takes three levels of the one-kernel search (more than 16,384 entries), a 40,000-token
    prefill crosses every run of its row, and the others end inside their last runs."""
    reqs = [Request(40000, 40000), Request(30000, 900), Request(25000, 1), Request(41000, 5000)]
    n = sum(q.n_new for q in reqs)
    return custom("many_runs", 4742, reqs, block_size=1, num_blocks=140000, runs=("len", 1, 1),
                  num_kv_heads=1, head_dim=64, max_num_tokens=n + 99)


SEARCH_CASES = [_short_prefills, _many_runs]


@pytest.mark.parametrize("variant", ["paged", "ranges"])
@pytest.mark.parametrize("make", SEARCH_CASES, ids=lambda f: f.__name__.strip("_"))
def test_slot_mapping_search_paths(make, variant):
    w = make()
    say(f"[slots] {w.describe()} {variant}")
    g, gf = gpu_slots(w, DeviceInputs(w), variant)
    o, of = oracle_slots(w, variant)
    assert np.array_equal(g, o) and gf == of == 0


@pytest.mark.parametrize("mode", WRITE_MODES)
@pytest.mark.parametrize("make", SEARCH_CASES, ids=lambda f: f.__name__.strip("_"))
def test_kv_write_search_paths(make, mode):
    check_kv_write(make(), mode)


_LC_PAYLOAD = {}


def long_context_payload():
    """The K/V payload of the 128K batch, on the host and on the device, drawn once from the
    R = 1 workload's seed and shared by the four layouts: they schedule the same requests and
    positions and differ only in block placement, so one payload serves them all (drawing
    2 x 256 MiB of bf16 takes about 25 s on the host)."""
    if not _LC_PAYLOAD:
        w = long_context(1)
        key_h, value_h = w.kv_plane(0), w.kv_plane(1)
        shape = (1, w.max_num_tokens, w.num_kv_heads, w.head_dim)
        _LC_PAYLOAD["host"] = (key_h, value_h)
        _LC_PAYLOAD["dev"] = (dev(key_h).view(shape), dev(value_h).view(shape))
    return _LC_PAYLOAD["host"], _LC_PAYLOAD["dev"]


@pytest.mark.parametrize("schedule", ["two", "one", "noslots"])
@pytest.mark.parametrize("variant", ["paged", "ranges_bs32", "ranges_expanded"])
@pytest.mark.parametrize("r", [1, 16, 512, 4096])
def test_kv_write_long_context(r, variant, schedule):
    """128K context, fused write of 131,072 tokens into an 8 GiB cache, whole cache compared
    byte for byte, at every range count: the block table expanded 32 -> 16 (paged), the
    manager-unit ranges at block size 32, and the ranges expanded to block size 16; with two
    kernels, with one kernel keeping the slot mapping, and with no slot-mapping output (one
    kernel under the automatic schedule)."""
    w = long_context(r)
    say(f"[kv_write long] {w.describe()} {variant} schedule={schedule}")
    orc = oracle.get()
    d = DeviceInputs(w)
    k = w.blocks_per_kv_block
    (key_h, value_h), (key, value) = long_context_payload()
    bs_k, nb_k = w.kernel_block_size, w.kernel_num_blocks
    suffix = "-" + schedule
    caches = Caches(1, nb_k, bs_k, w.row_elems)
    o_slots, o_flags = orc.slot_mapping_ranges(w.query_start_loc, w.num_reqs, w.positions,
                                               w.max_num_tokens, w.range_start, w.range_len,
                                               w.range_cum, w.num_ranges, w.block_size)
    assert o_flags == 0
    if variant == "paged":
        kt = torch.empty((w.max_num_reqs, w.table_stride * k), dtype=torch.int32, device=DEV)
        kvw.kvw_map_to_kernel_blocks(d.block_table, d.nbpr, w.block_size, bs_k, kt)
        sm, flags = run_kv_write(w, d, "paged" + suffix, caches, key, value, block_size=bs_k,
                                 num_blocks=nb_k, over=dict(block_table=kt, nbpr=d.nbpr * k))
    elif variant == "ranges_expanded":
        outs = [torch.empty_like(d.rs) for _ in range(3)] + [torch.empty_like(d.nr)]
        kvw.kvw_map_ranges_to_kernel_blocks(d.rs, d.rl, d.rc, d.nr, w.block_size, bs_k, *outs)
        sm, flags = run_kv_write(w, d, "ranges" + suffix, caches, key, value, block_size=bs_k,
                                 num_blocks=nb_k,
                                 over=dict(rs=outs[0], rl=outs[1], rc=outs[2], nr=outs[3]))
    else:
        sm, flags = run_kv_write(w, d, "ranges" + suffix, caches, key, value,
                                 block_size=w.block_size, num_blocks=w.num_blocks)
    assert (sm is None or np.array_equal(sm, o_slots)) and flags == 0
    # slots are identical in manager and kernel units, so one oracle pass checks every variant
    assert compare_caches(w, caches, o_slots, key_h, value_h, nb_k, bs_k) == 0


@pytest.mark.parametrize("mode", ["paged", "ranges", "paged-noslots", "ranges-noslots"])
def test_kv_write_32_layers(mode):
    """16,384 tokens x 32 layers in one launch into 2 x 32 GiB cache planes."""
    check_kv_write(config("full_32_layer"), mode)


# ---------------------------------------------------------------------------
# flags, padding and degenerate sizes
# ---------------------------------------------------------------------------
def _flagged_workload(heads=8, head_dim=128):
    reqs = [Request(100, 40), Request(70, 1), Request(300, 30), Request(20, 20)]
    w = custom("flagged", 4790, reqs, block_size=16, num_blocks=64, runs=("count", 1, 3),
               max_num_tokens=120, table_stride=24, range_stride=6, num_kv_heads=heads,
               head_dim=head_dim)
    w.num_blocks_per_req[0] = 99      # above the row width: clamped
    w.num_blocks_per_req[3] = -3      # negative: clamped to 0
    w.block_table[1, 4] = -7          # negative physical block (request 1 writes logical block 4)
    w.block_table[2, 16] = 900        # beyond the pool (request 2 writes logical blocks 16..18)
    # request 1: more ranges than the stride holds; fill the row with valid runs past its blocks
    n1 = int(w.num_ranges[1])
    end = int(w.range_cum[1, n1 - 1] + w.range_len[1, n1 - 1])
    for i in range(n1, w.range_stride):
        w.range_start[1, i], w.range_len[1, i], w.range_cum[1, i] = 40 + i, 1, end
        end += 1
    w.num_ranges[1] = 50
    w.num_ranges[3] = -1
    # request 2: the run holding logical block 17 starts below block 0
    for i in range(int(w.num_ranges[2])):
        if w.range_cum[2, i] <= 17 < w.range_cum[2, i] + w.range_len[2, i]:
            w.range_start[2, i] = -100
    return w


@pytest.mark.parametrize("variant", ["paged", "ranges"])
def test_flags_and_clamps(variant):
    w = _flagged_workload()
    d = DeviceInputs(w)
    g, gf = gpu_slots(w, d, variant)
    o, of = oracle_slots(w, variant)
    assert np.array_equal(g, o) and gf == of and of != 0
    # num_tokens past max_num_tokens
    q = w.query_start_loc.copy()
    q[-1] = w.max_num_tokens + 50
    d.qsl = dev(q)
    g, gf = gpu_slots(w, d, variant)
    o, of = oracle_slots(w, variant, qsl=q)
    assert np.array_equal(g, o) and gf == of and of & kvw.KVW_FLAG_NUM_TOKENS


# 2 KiB rows (the slice-granular scatter), 256 B and 48 B rows (several tokens per wave, each
# lane's row load issued with its slot load): padded, negative and out-of-pool slots alike
FLAG_ROWS = [(8, 128), (1, 128), (1, 24)]


@pytest.mark.parametrize("shape", FLAG_ROWS, ids=lambda s: f"{s[0] * s[1] * 2}B")
@pytest.mark.parametrize("mode", WRITE_MODES[1:])
def test_kv_write_flagged(mode, shape):
    check_kv_write(_flagged_workload(*shape), mode)


@pytest.mark.parametrize("shape", FLAG_ROWS, ids=lambda s: f"{s[0] * s[1] * 2}B")
def test_kv_write_out_of_pool_and_bad_slots(shape):
    w = _flagged_workload(*shape)
    # precomputed slots beyond the cache and below the pad id write nothing
    key_h = w.kv_plane(0)
    rng = np.random.default_rng(4)
    slots = np.full(w.max_num_tokens, -1, np.int64)
    rows = w.num_blocks * w.block_size
    slots[:60] = rng.permutation(rows)[:60]
    slots[60:70] = rows + np.arange(10)
    slots[70:75] = -(2 + np.arange(5))
    key = dev(key_h).view(1, w.max_num_tokens, w.num_kv_heads, w.head_dim)
    caches = Caches(1, w.num_blocks, w.block_size, w.row_elems)
    sm, flags = run_kv_write(w, DeviceInputs(w), "precomputed", caches, key, key, slots_in=slots)
    c_flags = compare_caches(w, caches, slots, key_h, key_h, w.num_blocks, w.block_size)
    assert flags == c_flags == kvw.KVW_FLAG_SLOT_OOB


def test_zero_token_rows_and_zero_layers():
    w = config("tiny_prefill")
    d = DeviceInputs(w)
    out = torch.full((4,), 9, dtype=torch.int64, device=DEV)
    kvw.kvw_slot_mapping_paged(d.qsl, w.num_reqs, d.positions, 0, d.block_table, d.nbpr, 16, out)
    torch.cuda.synchronize()
    assert host(out).tolist() == [9, 9, 9, 9]
    # fused call with no layers still produces the slot mapping and touches no cache
    key = torch.zeros((0, w.max_num_tokens, 8, 128), dtype=torch.int16, device=DEV)
    caches = Caches(1, 4, 16, 1024)
    sm = torch.full((w.max_num_tokens,), 5, dtype=torch.int64, device=DEV)
    kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_PAGED, key=key, value=key, k_cache=caches.k,
                     v_cache=caches.v, num_blocks=w.num_blocks, block_size=16,
                     max_num_tokens=w.max_num_tokens, query_start_loc=d.qsl,
                     num_reqs=w.num_reqs, positions=d.positions, block_table=d.block_table,
                     num_blocks_per_req=d.nbpr, slot_mapping_out=sm)
    o, _ = oracle_slots(w, "paged")
    torch.cuda.synchronize()
    assert np.array_equal(host(sm), o)
    assert (host(caches.t) == 0x7FC0).all()


@pytest.mark.parametrize("counts", [True, False], ids=["counts", "nocounts"])
@pytest.mark.parametrize("schedule", ["", "two", "one"])
def test_zero_width_block_table(schedule, counts):
    """A paged table of width 0 (no pointer): every token gets the pad id and nothing is
    written; with counts, every request whose count exceeds the width raises KVW_FLAG_COUNT."""
    w = config("tiny_prefill")
    d = DeviceInputs(w)
    table = torch.zeros((w.num_reqs, 0), dtype=torch.int32, device=DEV)
    key, value = kv_device(w)
    caches = Caches(w.num_layers, w.num_blocks, w.block_size, w.row_elems)
    sm = torch.full((w.max_num_tokens,), 7, dtype=torch.int64, device=DEV)
    flag = new_flag()
    kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_PAGED, key=key, value=value, k_cache=caches.k,
                     v_cache=caches.v, num_blocks=w.num_blocks, block_size=w.block_size,
                     query_start_loc=d.qsl, num_reqs=w.num_reqs, positions=d.positions,
                     block_table=table, num_blocks_per_req=d.nbpr if counts else None,
                     slot_mapping_out=sm, err_flag=flag, schedule=SCHEDULES[schedule])
    o, of = oracle_slots(w, "paged", block_table=np.zeros((w.num_reqs, 0), np.int32),
                         nbpr=w.num_blocks_per_req if counts else None)
    torch.cuda.synchronize()
    assert (o == -1).all() and np.array_equal(host(sm), o)
    assert int(flag.item()) == of == (kvw.KVW_FLAG_COUNT if counts else 0)
    assert (host(caches.t) == BF16_SENTINEL).all()


def test_invalid_arguments_raise():
    w = config("tiny_prefill")
    d = DeviceInputs(w)
    out = torch.empty(w.max_num_tokens, dtype=torch.int64, device=DEV)
    with pytest.raises(kvw.KvwError) as e:
        kvw.kvw_slot_mapping_paged(d.qsl, w.num_reqs, d.positions, w.max_num_tokens,
                                   d.block_table, d.nbpr, 0, out)
    assert e.value.status == 1
    kt = torch.empty((4, 64), dtype=torch.int32, device=DEV)
    with pytest.raises(kvw.KvwError):
        kvw.kvw_map_to_kernel_blocks(d.block_table, d.nbpr, 32, 12, kt)
    big = torch.zeros((4, kvw.kvw.KVW_MAX_RANGE_STRIDE + 1), dtype=torch.int32, device=DEV)
    with pytest.raises(kvw.KvwError) as e:
        kvw.kvw_slot_mapping_ranges(d.qsl, w.num_reqs, d.positions, w.max_num_tokens, big, big,
                                    big, d.nr, 16, out)
    assert e.value.status == 3
    # positions must hold max_num_tokens entries (the kernels read a padded token's too): the
    # binding refuses a shorter array before anything is launched
    short = d.positions[:w.max_num_tokens - 1]
    with pytest.raises(ValueError, match="fewer than max_num_tokens"):
        kvw.kvw_slot_mapping_paged(d.qsl, w.num_reqs, short, w.max_num_tokens, d.block_table,
                                   d.nbpr, w.block_size, out)
    key, value = kv_device(w)
    cache = torch.empty((w.num_blocks * w.block_size, w.row_elems), dtype=torch.int16, device=DEV)
    with pytest.raises(ValueError, match="fewer than max_num_tokens"):
        kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_RANGES, key=key, value=value, k_cache=cache,
                         v_cache=cache, num_blocks=w.num_blocks, block_size=w.block_size,
                         query_start_loc=d.qsl, num_reqs=w.num_reqs, positions=short,
                         range_start=d.rs, range_len=d.rl, range_cum=d.rc, num_ranges=d.nr)
