"""Graph capture: the fused write captured once at padded sizes, replayed with new batches.

Launch shapes depend only on host scalars (max_num_tokens, padded request
count, strides, layer count), so one captured graph serves every batch that
fits those sizes; the tail of the slot mapping and the rows of dummy requests
must come out as the pad id on every replay ("Blocktabelle" page,
"Datenfluss": the tail is padded so graph replay sees stable values).
The captured call also writes the attention side's block table at block
size 8.  Each replay is checked against the CPU oracle; caches are re-filled
eagerly between replays (no fill inside the graph).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_46_amd as kvw
from parity import DEV, Caches, compare_caches, dev, host, new_flag, oracle_slots, say
from workloads import custom
from workloads.gen import Request

pytestmark = pytest.mark.gpu

MAX_REQS, M, LAYERS, STRIDE, RSTRIDE, POOL = 12, 600, 2, 40, 8, 2048


def batch(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(4, MAX_REQS + 1))
    reqs, left = [], M - 20
    for _ in range(n):
        end = int(rng.integers(1, 600))
        new = int(min(end, rng.integers(1, 80), left))
        left -= new
        reqs.append(Request(end, new))
    return custom(f"graph_batch_{seed}", seed, reqs, block_size=16, num_blocks=POOL,
                  runs=("count", 1, 4), num_layers=LAYERS, max_num_tokens=M, table_stride=STRIDE,
                  range_stride=RSTRIDE, dummy_reqs=MAX_REQS - n)


@pytest.mark.parametrize("keep_slots", [True, False], ids=["slots", "noslots"])
@pytest.mark.parametrize("variant", ["paged", "ranges"])
def test_graph_replay_matches_oracle(variant, keep_slots):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    batches = [batch(4800 + i) for i in range(3)]
    w0 = batches[0]
    # static device buffers at the padded sizes
    static = {name: dev(getattr(w0, name)) for name in
              ("query_start_loc", "positions", "block_table", "num_blocks_per_req",
               "range_start", "range_len", "range_cum", "num_ranges")}
    key = torch.empty((LAYERS, M, w0.num_kv_heads, w0.head_dim), dtype=torch.int16, device=DEV)
    value = torch.empty_like(key)
    caches = Caches(LAYERS, POOL, 16, w0.row_elems)
    sm = torch.full((M,), 31, dtype=torch.int64, device=DEV)
    # the attention side's table at block size 8, written by the same launches
    table = torch.full((MAX_REQS, STRIDE * 2), -5, dtype=torch.int32, device=DEV)
    counts = torch.full((MAX_REQS,), -5, dtype=torch.int32, device=DEV)
    flag = new_flag()
    mode = kvw.KVW_SLOTS_PAGED if variant == "paged" else kvw.KVW_SLOTS_RANGES
    mapping = (dict(block_table=static["block_table"],
                    num_blocks_per_req=static["num_blocks_per_req"]) if variant == "paged" else
               dict(range_start=static["range_start"], range_len=static["range_len"],
                    range_cum=static["range_cum"], num_ranges=static["num_ranges"]))

    def load(w):
        for name, t in static.items():
            t.copy_(dev(getattr(w, name)))
        key.copy_(dev(w.kv_plane(0)).view_as(key))
        value.copy_(dev(w.kv_plane(1)).view_as(value))
        caches.t.fill_(0x7FC0)
        sm.fill_(31)
        table.fill_(-5)
        counts.fill_(-5)
        flag.zero_()

    def call():
        kvw.kvw_kv_write(mode=mode, key=key, value=value, k_cache=caches.k, v_cache=caches.v,
                         num_blocks=POOL, block_size=16, max_num_tokens=M,
                         query_start_loc=static["query_start_loc"], num_reqs=MAX_REQS,
                         positions=static["positions"],
                         slot_mapping_out=sm if keep_slots else None, err_flag=flag,
                         table_out=table, table_counts_out=counts, table_block_size=8, **mapping)

    load(w0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for rep, w in enumerate(batches + batches[:1]):
        say(f"[graph] {variant} keep_slots={keep_slots} replay {rep}: {w.describe()}")
        load(w)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_slots, o_flags = oracle_slots(w, variant)
        if keep_slots:
            assert np.array_equal(host(sm), o_slots)
            assert (host(sm)[w.num_tokens:] == -1).all()
        c_flags = compare_caches(w, caches, o_slots, w.kv_plane(0), w.kv_plane(1), POOL, 16)
        orc = oracle.get()
        if variant == "paged":
            o_t, o_c, t_flags = orc.map_to_kernel_blocks(w.block_table, w.num_blocks_per_req, 16, 8,
                                                         with_counts=True)
        else:
            o_t, o_c, t_flags = orc.ranges_to_block_table(w.range_start, w.range_len, w.range_cum,
                                                          w.num_ranges, 16, 8, STRIDE * 2)
        assert np.array_equal(host(table), o_t) and np.array_equal(host(counts), o_c)
        assert int(flag.item()) == o_flags | c_flags | t_flags == 0
