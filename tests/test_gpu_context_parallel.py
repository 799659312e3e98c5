"""Context-parallel slot mapping and K/V write: HIP path vs CPU oracle (needs an MI355X).

Each workload's block size is the virtual block of W ranks; each rank's cache
holds blocks of block_size / W slots.  Every rank is run in turn on the one
GPU, with its own cache.  Slots and flags are compared exactly, caches byte
for byte, and over the ranks every real token must be written exactly once.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_46_amd as kvw
from parity import DEV, Caches, DeviceInputs, compare_caches, dev, host, new_flag, say
from workloads import config, long_context, small_cases

pytestmark = pytest.mark.gpu

SMALL = {w.name: w for w in small_cases()}
# (workload, W, interleave sizes): block sizes 64, 16, 16 split into 2 to 8 ranks
SLOT_CASES = [("small_bs64", 2, (1, 32)), ("small_bs64", 4, (1, 4, 16)), ("small_bs64", 8, (1, 8)),
              ("tiny_prefill", 2, (1, 4, 8)), ("small_mixed_l3", 4, (1, 2, 4)),
              ("small_dummy", 2, (8,)), ("small_out_of_range", 2, (1,)),
              ("decode_step", 2, (1, 8)), ("mixed_chunked", 4, (1, 4))]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvw.library()
    yield
    torch.cuda.synchronize()


def workload(name):
    return SMALL[name] if name in SMALL else config(name)


def oracle_cp(w, variant, world, rank, interleave):
    orc = oracle.get()
    bs = w.block_size // world
    if variant == "paged":
        return orc.slot_mapping_paged_cp(w.query_start_loc, w.num_reqs, w.positions,
                                         w.max_num_tokens, w.block_table, w.num_blocks_per_req,
                                         bs, world, rank, interleave)
    return orc.slot_mapping_ranges_cp(w.query_start_loc, w.num_reqs, w.positions,
                                      w.max_num_tokens, w.range_start, w.range_len, w.range_cum,
                                      w.num_ranges, bs, world, rank, interleave)


def gpu_cp(w, d, variant, world, rank, interleave):
    out = torch.full((w.max_num_tokens,), 12345, dtype=torch.int64, device=DEV)
    flag = new_flag()
    bs = w.block_size // world
    cp = dict(cp_world_size=world, cp_rank=rank, cp_interleave_size=interleave)
    if variant == "paged":
        kvw.kvw_slot_mapping_paged(d.qsl, w.num_reqs, d.positions, w.max_num_tokens,
                                   d.block_table, d.nbpr, bs, out, flag, **cp)
    else:
        kvw.kvw_slot_mapping_ranges(d.qsl, w.num_reqs, d.positions, w.max_num_tokens, d.rs, d.rl,
                                    d.rc, d.nr, bs, out, flag, **cp)
    torch.cuda.synchronize()
    return host(out), int(flag.item())


@pytest.mark.parametrize("variant", ["paged", "ranges"])
@pytest.mark.parametrize("case", SLOT_CASES, ids=lambda c: f"{c[0]}-W{c[1]}")
def test_cp_slot_mapping(case, variant):
    name, world, interleaves = case
    w = workload(name)
    d = DeviceInputs(w)
    for interleave in interleaves:
        held = np.zeros(w.max_num_tokens, np.int64)
        for rank in range(world):
            say(f"[cp slots] {name} {variant} W={world} I={interleave} rank={rank}")
            g, gf = gpu_cp(w, d, variant, world, rank, interleave)
            o, of = oracle_cp(w, variant, world, rank, interleave)
            bad = np.nonzero(g != o)[0]
            assert len(bad) == 0, f"{len(bad)} slots differ, first token {bad[:4].tolist()}"
            assert gf == of
            held += g >= 0
        assert held.max() <= 1


@pytest.mark.parametrize("variant", ["paged", "ranges"])
def test_cp_long_context(variant):
    """128K context, manager blocks of 32 = virtual blocks of two ranks of 16-slot blocks."""
    w = long_context(4096)
    d = DeviceInputs(w)
    for interleave in (1, 16):
        real = 0
        for rank in range(2):
            say(f"[cp slots] {w.name} {variant} W=2 I={interleave} rank={rank}")
            g, gf = gpu_cp(w, d, variant, 2, rank, interleave)
            o, of = oracle_cp(w, variant, 2, rank, interleave)
            assert np.array_equal(g, o) and gf == of == 0
            real += int((g >= 0).sum())
        assert real == w.num_tokens


CP_WRITE_MODES = ["paged", "ranges", "paged-two", "ranges-two", "paged-one", "ranges-one",
                  "paged-noslots", "ranges-noslots"]
SCHEDULES = {"": kvw.KVW_SCHEDULE_AUTO, "two": kvw.KVW_SCHEDULE_TWO_KERNELS,
             "one": kvw.KVW_SCHEDULE_ONE_KERNEL, "noslots": kvw.KVW_SCHEDULE_AUTO}


def cp_write_and_compare(w, mode, world, interleave):
    variant, _, sched = mode.partition("-")
    d = DeviceInputs(w)
    bs = w.block_size // world
    key_h, value_h = w.kv_plane(0), w.kv_plane(1)
    key = dev(key_h).view(w.num_layers, w.max_num_tokens, w.num_kv_heads, w.head_dim)
    value = dev(value_h).view_as(key)
    written = np.zeros(w.max_num_tokens, np.int64)
    for rank in range(world):
        say(f"[cp write] {w.describe()} mode={mode} W={world} I={interleave} rank={rank}")
        o_slots, o_flags = oracle_cp(w, variant, world, rank, interleave)
        caches = Caches(w.num_layers, w.num_blocks, bs, w.row_elems)
        flag = new_flag()
        sm = torch.full((w.max_num_tokens,), 777, dtype=torch.int64, device=DEV)
        kw = dict(query_start_loc=d.qsl, num_reqs=w.num_reqs, positions=d.positions,
                  slot_mapping_out=None if sched == "noslots" else sm)
        if variant == "paged":
            kw.update(mode=kvw.KVW_SLOTS_PAGED, block_table=d.block_table,
                      num_blocks_per_req=d.nbpr)
        else:
            kw.update(mode=kvw.KVW_SLOTS_RANGES, range_start=d.rs, range_len=d.rl,
                      range_cum=d.rc, num_ranges=d.nr)
        kvw.kvw_kv_write(key=key, value=value, k_cache=caches.k, v_cache=caches.v,
                         num_blocks=w.num_blocks, block_size=bs, max_num_tokens=w.max_num_tokens,
                         err_flag=flag, schedule=SCHEDULES[sched], cp_world_size=world,
                         cp_rank=rank, cp_interleave_size=interleave, **kw)
        torch.cuda.synchronize()
        if sched != "noslots":
            assert np.array_equal(host(sm), o_slots)
        c_flags = compare_caches(w, caches, o_slots, key_h, value_h, w.num_blocks, bs)
        assert int(flag.item()) == o_flags | c_flags
        written += o_slots >= 0
        del caches
    return written


@pytest.mark.parametrize("mode", CP_WRITE_MODES)
@pytest.mark.parametrize("case", [("small_bs64", 4, 16), ("tiny_prefill", 2, 1),
                                  ("small_mixed_l3", 2, 4)], ids=lambda c: f"{c[0]}-W{c[1]}")
def test_cp_kv_write(case, mode):
    name, world, interleave = case
    w = workload(name)
    written = cp_write_and_compare(w, mode, world, interleave)
    assert written.max() <= 1


@pytest.mark.parametrize("mode", ["paged", "ranges-noslots"])
def test_cp_kv_write_long_context(mode):
    w = long_context(4096)
    written = cp_write_and_compare(w, mode, 2, 16)
    assert written.sum() == w.num_tokens and written.max() == 1


def test_cp_flags():
    """Clamped counts, negative blocks and an over-long range count, under context parallelism."""
    from test_gpu_parity import _flagged_workload
    w = _flagged_workload()
    d = DeviceInputs(w)
    seen = 0
    for variant in ("paged", "ranges"):
        for rank in range(2):
            say(f"[cp flags] {variant} rank={rank}")
            g, gf = gpu_cp(w, d, variant, 2, rank, 2)
            o, of = oracle_cp(w, variant, 2, rank, 2)
            assert np.array_equal(g, o) and gf == of
            seen |= of
    assert seen & kvw.KVW_FLAG_COUNT and seen & kvw.KVW_FLAG_BAD_BLOCK
