"""Benchmark of the fused slot-map + K/V write on one MI355X.

Default workload: 128K context, 16 requests x 8192-token prefill chunks
(131,072 tokens written per step), manager block size 32 expanded to kernel
block size 16, 8 KV heads x 128 bf16, one layer.  Each request's blocks form
R contiguous runs placed at random (R in 1, 16, 512, 4096; 4096 = every
manager block on its own).  A step is the whole hot path for one batch:
manager->kernel expansion of the variant's mapping structure, then the fused
slot-map + K/V write (kvw_kv_write keeping the slot mapping, automatic
kernel schedule) on the manager-unit mapping: slot ids are the same at
either block size.  Both variants hand the attention side the same
kernel-unit block table, written by extra workgroups of the slot-mapping
launch (kvw_kv_write's table_out), so a step is two launches:

  paged_r{R}     manager block table expanded, fused paged write
  ranges_r{R}    block table filled straight from the range descriptors,
                 fused range write

"fused call" times the write without the table.  The table-producing kernel
of each variant is also timed alone (as its own call), next to a plain
device copy of the finished table (the per-step copy of a staged table that
the fill replaces).  On the headline layout, the fused write is
also timed per context-parallel rank (two ranks, interleave 1 and 16): each
rank writes its share of the batch into its own cache.  And per
tensor-parallel rank (TP = 2, 4, 8 over the 8 KV heads): rows of 2048/TP
bytes, every token.

The read side is measured too ("decode_attention"): decode attention, one
query per request with 32 query heads over the 8 KV heads, over the 128K
layouts (R = 1 and 4096) and the 256-request decode step, paged gather vs
range arithmetic, at every chunk length; the R = 1 layout also with 8, 16
and 64 query heads (1, 2 and 8 per KV head); and decode context parallelism
at W = 2 (each rank's share, then the log-sum-exp merge).  Each decode
workload opens with half a second of untimed calls.  --decode-only runs just
that part (for profiling).

`value` is tokens/s of paged_r4096; every variant is reported under
"variants", with the fused call's time (HIP events on the launch stream)
and the time of the one-kernel schedule.
The roofline entry is for kv_scatter_kernel, the dominant kernel, timed
alone on the headline variant's slots.  The CPU baseline times the CPU
oracle (test infrastructure) on the same batch.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s and HBM GB/s (% of peak) for fused slot-map+KV write, paged vs range"
# headline: paged gather over the fully fragmented layout (every manager block its own run)
HEADLINE = "paged_r4096"
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_46_amd", "csrc", "kvw.hip"),
                  os.path.join(ROOT, "paged_kv_cache_46_amd", "csrc", "kvw_device.h"),
                  os.path.join(ROOT, "include", "kvw.h")]
COUNTERS = os.path.join(ROOT, "profiles", "kv_scatter_kernel_long_context_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--variants", default=",".join(
        f"{k}_r{r}" for k in ("paged", "ranges") for r in (1, 16, 512, 4096)))
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the CPU oracle timing (e.g. under a profiler)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--workload", default="long_context",
                   choices=["long_context", "tiny_prefill", "decode_step", "mixed_chunked",
                            "full_32_layer"],
                   help="long_context (default) is the 128K study above; the others time the\n"
                        "fused write (paged and ranges) on that config, flushing L2 and MALL\n"
                        "before every step; ms_per_step is then the fused call's event time")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the decode-attention (read path) measurements")
    p.add_argument("--decode-only", action="store_true",
                   help="run only the decode-attention measurements (for profiling); prints\n"
                        "their JSON object instead of the benchmark line")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other four study configs (reported under \"configs\")")
    p.add_argument("--slot-mapping-only", action="store_true",
                   help="run only the slot mapping, paged then ranges, 10 calls each with L2 and\n"
                        "MALL evicted before every call, on the 128K layouts (R = 1, 16, 512,\n"
                        "4096; manager units), the decode step and the mixed batch, in that order\n"
                        "(for hardware-counter profiles); prints the order of the calls as JSON")
    p.add_argument("--copy-calibration-mib", type=int, default=512,
                   help="size of the plain device copy timed as the practical ceiling "
                        "(read + write of this many MiB); 0 to skip")
    return p.parse_args()


def kernel_source_hash() -> str:
    """sha256 of the write path's device source (kvw.hip, kvw_device.h and kvw.h) with comments,
    trailing blanks and empty lines removed: what the compiled kernels depend on, so that an
    edited comment does not void counters taken on the same code."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines()]
        h.update(os.path.basename(path).encode())
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()


def counter_traffic():
    """HBM bytes per fused-write launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on a different kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return c.get("traffic_bytes_per_launch")


def timed(fn, n_warm, n_steps):
    """Wall ms per call over n_steps bare calls (between two synchronizations), then the
    per-call HIP-event times of a second, instrumented pass of n_steps calls (the event
    records cost the stream a few microseconds, so they stay out of the wall time)."""
    import torch
    for _ in range(n_warm):
        fn(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_steps):
        fn(None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_steps)]
    torch.cuda.synchronize()
    for i in range(n_steps):
        fn(evs[i])
    torch.cuda.synchronize()
    return wall * 1e3 / n_steps, [a.elapsed_time(b) for a, b in evs]


def timed_block(fn, n_warm, n_steps):
    """Average ms per call of n_steps back-to-back calls between one pair of HIP events on the
    launch stream: a kernel's steady-state launch duration, without the cost of an event pair
    around each call (a few microseconds)."""
    import torch
    for _ in range(n_warm):
        fn(None)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(torch.cuda.current_stream())
    for _ in range(n_steps):
        fn(None)
    e1.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n_steps


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; multi-GPU runs are not part of it "
              "(the write path shards with no exchange step: each GPU writes its own cache shard)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_46_amd as kvw
    from workloads import BF16_SENTINEL, long_context

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    kvw.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.slot_mapping_only:
        print(json.dumps(slot_mapping_only()), flush=True)
        return
    if args.workload != "long_context":
        bench_config(args)
        return
    if args.decode_only:
        def d_(a):
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        print(json.dumps(decode_attention(args, d_, dev, torch.cuda.current_stream(), timed)),
              flush=True)
        return

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    variants = [v for v in args.variants.split(",") if v]
    base = long_context(1)
    M, H, D = base.max_num_tokens, base.num_kv_heads, base.head_dim
    bpt = base.bytes_per_token
    k = base.blocks_per_kv_block
    bs_k, nb_k = base.kernel_block_size, base.kernel_num_blocks
    log(f"[bench] workload {base.describe()} -> kernel bs {bs_k}, {nb_k} kernel blocks")
    t = time.time()
    # one K/V payload serves every layout variant (same requests and positions)
    key = d(base.kv_layer(0, 0)).view(1, M, H, D)
    value = d(base.kv_layer(1, 0)).view(1, M, H, D)
    log(f"[bench] K/V generated and uploaded in {time.time() - t:.1f}s "
        f"({2 * M * bpt / 2**20:.0f} MiB)")
    cache = torch.full((2, nb_k * bs_k, H * D), BF16_SENTINEL, dtype=torch.int16, device=dev)
    sm_out = torch.empty(M, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()

    # algorithmic bytes of the fused write per launch: K and V rows read and written
    # (4 x bytes_per_token per token per layer) + position read + slot written (8 + 8 B)
    real_tokens = base.num_tokens
    fused_bytes = real_tokens * base.num_layers * 4 * bpt + real_tokens * 16
    # the scatter kernel alone: K and V rows read and written + slot read (8 B)
    scatter_bytes = real_tokens * base.num_layers * 4 * bpt + real_tokens * 8

    results = {}
    scatter = scatter_pairs = contiguous_ms = None
    for name in variants:
        kind, _, r = name.partition("_r")
        if kind not in ("paged", "ranges") or not r.isdigit():
            raise SystemExit(f"unknown variant {name}")
        w = long_context(int(r))
        qsl, pos = d(w.query_start_loc), d(w.positions)
        # Slot ids do not change under manager->kernel expansion (same memory at a finer
        # block size), so the write takes the manager-unit mapping; the expansion's output is
        # for the attention side.  (Running the expansion on a second stream was measured
        # slower: the cross-stream waits cost more than the 4 us kernel they would hide.)
        if kind == "paged":
            bt, nb = d(w.block_table), d(w.num_blocks_per_req)
            kt = torch.empty((w.max_num_reqs, w.table_stride * k), dtype=torch.int32, device=dev)
            kn = torch.empty_like(nb)
            expand_bytes = (w.block_table.nbytes + w.num_blocks_per_req.nbytes + kt.numel() * 4
                            + kn.numel() * 4)
            mapping = dict(block_table=bt, num_blocks_per_req=nb)

            def expand(bt=bt, nb=nb, kt=kt, w=w):
                kvw.kvw_map_to_kernel_blocks(bt, nb, w.block_size, bs_k, kt)  # no counts here
            mode = kvw.KVW_SLOTS_PAGED
        else:
            rs, rl, rc, nr = (d(a) for a in (w.range_start, w.range_len, w.range_cum, w.num_ranges))
            kt = torch.empty((w.max_num_reqs, w.table_stride * k), dtype=torch.int32, device=dev)
            kn = torch.empty_like(nr)
            # descriptors read (12 B per run in use + the count) + table and counts written
            expand_bytes = (12 * int(w.num_ranges.sum()) + w.num_ranges.nbytes + kt.numel() * 4
                            + kn.numel() * 4)
            mapping = dict(range_start=rs, range_len=rl, range_cum=rc, num_ranges=nr)

            def expand(rs=rs, rl=rl, rc=rc, nr=nr, kt=kt, kn=kn, w=w):
                kvw.kvw_ranges_to_block_table(rs, rl, rc, nr, w.block_size, bs_k, kt, kn)
            mode = kvw.KVW_SLOTS_RANGES

        def write(schedule, table=False, mode=mode, mapping=mapping, qsl=qsl, pos=pos, w=w,
                  kt=kt, kn=kn):
            extra = dict(table_out=kt, table_counts_out=kn, table_block_size=bs_k) if table else {}
            kvw.kvw_kv_write(mode=mode, key=key, value=value, k_cache=cache[0], v_cache=cache[1],
                             num_blocks=w.num_blocks, block_size=w.block_size,
                             query_start_loc=qsl, num_reqs=w.num_reqs, positions=pos,
                             slot_mapping_out=sm_out, schedule=schedule, **mapping, **extra)

        def step(ev, write=write):
            # the whole step: slots + attention-side table in one launch, then the scatter
            if ev is not None:
                ev[0].record(stream)
            write(kvw.KVW_SCHEDULE_AUTO, table=True)
            if ev is not None:
                ev[1].record(stream)

        def fused_call(ev, write=write):
            if ev is not None:
                ev[0].record(stream)
            write(kvw.KVW_SCHEDULE_AUTO)
            if ev is not None:
                ev[1].record(stream)

        def single(ev, write=write):
            if ev is not None:
                ev[0].record(stream)
            write(kvw.KVW_SCHEDULE_ONE_KERNEL)
            if ev is not None:
                ev[1].record(stream)

        def table_only(ev, expand=expand):
            if ev is not None:
                ev[0].record(stream)
            expand()
            if ev is not None:
                ev[1].record(stream)

        def table_copy(ev, kt=kt):
            # a plain device copy of the finished table: what a staged table costs per step
            if ev is not None:
                ev[0].record(stream)
            table_dst.copy_(kt)
            if ev is not None:
                ev[1].record(stream)

        table_dst = torch.empty_like(kt)
        ms_step, step_ev_ms = timed(step, args.warmup, args.steps)
        _, call_ms = timed(fused_call, args.warmup, args.steps)
        call_avg = timed_block(fused_call, 0, args.steps)
        _, single_ms = timed(single, args.warmup, args.steps)
        single_avg = timed_block(single, 0, args.steps)
        _, table_ms = timed(table_only, args.warmup, args.steps)
        _, copy_ms = timed(table_copy, args.warmup, args.steps)
        table_avg = statistics.fmean(table_ms)
        copy_avg = statistics.fmean(copy_ms)
        step_bytes = fused_bytes + expand_bytes
        results[name] = {
            "tokens_per_s": real_tokens / (ms_step * 1e-3),
            "ms_per_step": ms_step,
            "step_event_ms_avg": statistics.fmean(step_ev_ms),
            "step_gbps": step_bytes / (ms_step * 1e-3) / 1e9,
            "call_timing": (f"{args.steps} calls back to back between one pair of HIP events; "
                            "*_event_pair_each: an event pair around each call"),
            "fused_call_ms_avg": call_avg,
            "fused_call_ms_event_pair_each": statistics.fmean(call_ms),
            "fused_call_event_pair_ms_p10": float(np.percentile(call_ms, 10)),
            "fused_call_event_pair_ms_p90": float(np.percentile(call_ms, 90)),
            "fused_call_gbps": fused_bytes / (call_avg * 1e-3) / 1e9,
            "fused_call_frac_of_peak": fused_bytes / (call_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "single_kernel_ms_avg": single_avg,
            "single_kernel_ms_event_pair_each": statistics.fmean(single_ms),
            "single_kernel_frac_of_peak": fused_bytes / (single_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "ranges_per_request": int(r),
            "table_kernel": "expand_blocks_kernel" if kind == "paged" else "fill_table_kernel",
            "table_ms_avg": table_avg,
            "table_bytes": expand_bytes,
            "table_gbps": expand_bytes / (table_avg * 1e-3) / 1e9,
            "table_copy_ms_avg": copy_avg,
        }
        log(f"[bench] {name:13s} step {ms_step * 1e3:7.1f} us  fused call {call_avg * 1e3:7.1f} us = "
            f"{results[name]['fused_call_gbps']:5.0f} GB/s "
            f"({100 * results[name]['fused_call_frac_of_peak']:.1f}%)  single kernel "
            f"{single_avg * 1e3:7.1f} us ({100 * results[name]['single_kernel_frac_of_peak']:.1f}%)  "
            f"{results[name]['tokens_per_s'] / 1e6:.0f} M tokens/s")
        log(f"[bench] {name:13s} {results[name]['table_kernel']} {table_avg * 1e3:6.2f} us "
            f"({expand_bytes / 1e6:.2f} MB, {results[name]['table_gbps']:.0f} GB/s); "
            f"device copy of the finished table {copy_avg * 1e3:6.2f} us")
        if name == HEADLINE:
            # the dominant kernel alone, on the slots the fused call just produced
            step(None)
            torch.cuda.synchronize()
            slots = sm_out.clone()

            def scatter_only(ev, slots=slots, w=w):
                if ev is not None:
                    ev[0].record(stream)
                kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_PRECOMPUTED, key=key, value=value,
                                 k_cache=cache[0], v_cache=cache[1], num_blocks=w.num_blocks,
                                 block_size=w.block_size, slot_mapping_in=slots)
                if ev is not None:
                    ev[1].record(stream)
            _, sc_ms = timed(scatter_only, args.warmup, args.steps)
            scatter_pairs = statistics.fmean(sc_ms)
            scatter = timed_block(scatter_only, 2, args.steps)  # warm already
            log(f"[bench] kv_scatter_kernel alone ({name} slots): {scatter * 1e3:.1f} us = "
                f"{scatter_bytes / (scatter * 1e-3) / 1e9:.0f} GB/s ({args.steps} launches back to "
                f"back; {scatter_pairs * 1e3:.1f} us with an event pair around each)")
            # The same copy kernel with the destination made contiguous (slot t for token t):
            # the rate this 16-byte copy (non-temporal loads, write-through stores) reaches
            # without the scattered blocks.
            ident = torch.arange(M, dtype=torch.int64, device=dev)

            def contiguous(ev, ident=ident, w=w):
                if ev is not None:
                    ev[0].record(stream)
                kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_PRECOMPUTED, key=key, value=value,
                                 k_cache=cache[0], v_cache=cache[1], num_blocks=w.num_blocks,
                                 block_size=w.block_size, slot_mapping_in=ident)
                if ev is not None:
                    ev[1].record(stream)
            contiguous_ms = timed_block(contiguous, args.warmup, args.steps)
            log(f"[bench] the same copy to a contiguous destination: {contiguous_ms * 1e3:.1f} us = "
                f"{scatter_bytes / (contiguous_ms * 1e-3) / 1e9:.0f} GB/s")
        del step, fused_call, single, write, expand, table_only, table_copy, table_dst

    # Context parallelism on the headline layout: the manager's 32-token blocks are the virtual
    # blocks of two ranks holding 16-slot blocks each; every rank writes its share of the batch
    # into its own cache (here a view of the same allocation), one rank after the other.
    cp = None
    if HEADLINE in results:
        w = long_context(int(HEADLINE.partition("_r")[2]))
        qsl, pos = d(w.query_start_loc), d(w.positions)
        bt, nb = d(w.block_table), d(w.num_blocks_per_req)
        world, bs_r = 2, w.block_size // 2
        rows = w.num_blocks * bs_r
        cp = {}
        for inter in (1, bs_r):
            for rank in range(world):
                def cp_call(ev, inter=inter, rank=rank):
                    if ev is not None:
                        ev[0].record(stream)
                    kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_PAGED, key=key, value=value,
                                     k_cache=cache[0, :rows], v_cache=cache[1, :rows],
                                     num_blocks=w.num_blocks, block_size=bs_r,
                                     query_start_loc=qsl, num_reqs=w.num_reqs, positions=pos,
                                     block_table=bt, num_blocks_per_req=nb,
                                     slot_mapping_out=sm_out, cp_world_size=world, cp_rank=rank,
                                     cp_interleave_size=inter)
                    if ev is not None:
                        ev[1].record(stream)
                _, cp_ms = timed(cp_call, args.warmup, args.steps)
                held = int((sm_out >= 0).sum().item())  # this rank's tokens, from its own output
                avg = timed_block(cp_call, 0, args.steps)
                rank_bytes = held * base.num_layers * 4 * bpt + M * 16
                cp[f"W{world}_I{inter}_rank{rank}"] = {
                    "tokens": held, "fused_call_ms_avg": round(avg, 6),
                    "fused_call_ms_event_pair_each": round(statistics.fmean(cp_ms), 6),
                    "gbps": round(rank_bytes / (avg * 1e-3) / 1e9, 1),
                    "frac_of_peak": round(rank_bytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
                log(f"[bench] context parallel W={world} I={inter:2d} rank {rank}: {held} tokens, "
                    f"fused call {avg * 1e3:6.1f} us = {cp[f'W{world}_I{inter}_rank{rank}']['gbps']:.0f}"
                    f" GB/s")
        del cp_call

    # Tensor parallelism over KV heads: a rank writes 8/TP heads of every token, so its rows
    # shrink to 2048/TP bytes; same layout, one rank's share measured.  A rank's write is small
    # enough (64-256 MB) for the memory-side cache to hold much of it, so consecutive calls take
    # four block tables in turn, the headline's with every block id shifted by a quarter of the
    # pool: no call rewrites the lines the call before wrote.
    tp = None
    if HEADLINE in results:
        tp = {}
        w = long_context(int(HEADLINE.partition("_r")[2]))
        qsl, pos = d(w.query_start_loc), d(w.positions)
        nb = d(w.num_blocks_per_req)
        quarter = w.num_blocks // 4
        bts = [d(((w.block_table.astype(np.int64) + k * quarter) % w.num_blocks).astype(np.int32))
               for k in range(4)]
        turn = [0]
        for tpn in (2, 4, 8):
            h = H // tpn
            k_r = key[:, :, :h, :].contiguous()
            v_r = value[:, :, :h, :].contiguous()
            rows = w.num_blocks * w.block_size
            k_c = cache[0].view(-1)[:rows * h * D].view(rows, h * D)
            v_c = cache[1].view(-1)[:rows * h * D].view(rows, h * D)

            def tp_call(ev, k_r=k_r, v_r=v_r, k_c=k_c, v_c=v_c):
                bt = bts[turn[0] % 4]
                turn[0] += 1
                if ev is not None:
                    ev[0].record(stream)
                kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_PAGED, key=k_r, value=v_r, k_cache=k_c,
                                 v_cache=v_c, num_blocks=w.num_blocks, block_size=w.block_size,
                                 query_start_loc=qsl, num_reqs=w.num_reqs, positions=pos,
                                 block_table=bt, num_blocks_per_req=nb, slot_mapping_out=sm_out)
                if ev is not None:
                    ev[1].record(stream)
            _, tp_ms = timed(tp_call, args.warmup, args.steps)
            avg = timed_block(tp_call, 0, args.steps)
            rank_bytes = real_tokens * base.num_layers * 4 * (bpt // tpn) + real_tokens * 16
            tp[f"TP{tpn}"] = {"bytes_per_token": bpt // tpn, "destinations": "4 block tables in turn",
                              "fused_call_ms_avg": round(avg, 6),
                              "fused_call_ms_event_pair_each": round(statistics.fmean(tp_ms), 6),
                              "gbps": round(rank_bytes / (avg * 1e-3) / 1e9, 1),
                              "frac_of_peak": round(rank_bytes / (avg * 1e-3) / 1e9
                                                    / HBM_PEAK_GBPS, 4)}
            log(f"[bench] tensor parallel TP={tpn} ({bpt // tpn} B rows): fused call "
                f"{avg * 1e3:6.1f} us = {tp[f'TP{tpn}']['gbps']:.0f} GB/s")
            del tp_call, k_r, v_r

    configs = None
    if not args.no_configs:
        configs = {name: config_results(name, args.steps, args.warmup,
                                        graph=name in GRAPH_CONFIGS) for name in STUDY_CONFIGS}

    dec = None
    if not args.no_decode:
        dec = decode_attention(args, d, dev, stream, timed, planes=cache)
    del cache

    copy_ceiling = None
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        reps = 20
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        copy_ceiling = {"torch_copy": {"what": "torch device-to-device copy_", "bytes_moved": 2 * n,
                                       "ms": ms, "gbps": 2 * n / (ms * 1e-3) / 1e9}}
        log(f"[bench] device copy of {args.copy_calibration_mib} MiB: {copy_ceiling['torch_copy']['gbps']:.0f} GB/s "
            "(read + write)")
        del src, dst

    if contiguous_ms is not None:
        copy_ceiling = copy_ceiling or {}
        copy_ceiling.update({
            "what": ("kv_scatter_kernel (16-byte non-temporal loads, non-temporal stores written "
                     "through L2, one 1 KiB slice per wave) on the headline batch with slot t for "
                     "token t: the step's copy with a contiguous destination"),
            "bytes_per_launch": scatter_bytes, "ms": round(contiguous_ms, 6),
            "gbps": round(scatter_bytes / (contiguous_ms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(scatter_bytes / (contiguous_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "same_kernel_step_slots_gbps": round(scatter_bytes / (scatter * 1e-3) / 1e9, 1)})

    host_alloc = host_allocator()

    cpu = cpu_par = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(long_context(int(HEADLINE.partition("_r")[2])), args.cpu_seconds)
        cpu_par = cpu_baseline_threads(long_context(int(HEADLINE.partition("_r")[2])),
                                       args.cpu_seconds / 3)

    head = results.get(HEADLINE) or next(iter(results.values()))
    traffic = counter_traffic()
    roof = None
    if scatter is not None:
        roof = {
            "bound": "hbm",
            "achieved": round(scatter_bytes / (scatter * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(scatter_bytes / (scatter * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "kv_scatter_kernel<1>",
            "launch_ms_avg": round(scatter, 5),
            "launch_timing": (f"{args.steps} launches back to back between one pair of HIP events "
                              "on the launch stream, after the step's own timing"),
            "launch_ms_avg_event_pair_each": round(scatter_pairs, 5),
            "algorithmic_bytes_per_launch": scatter_bytes,
        }
    line = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": "long_context_128k", "requests": base.num_reqs,
                   "tokens_per_step": real_tokens, "context": 131072, "layers": base.num_layers,
                   "manager_block_size": base.block_size, "kernel_block_size": bs_k,
                   "kv_heads": H, "head_dim": D, "payload": "bf16", "variant": HEADLINE},
        "hbm_gbps": round(head["step_gbps"], 1),
        "hbm_frac_of_peak": round(head["step_gbps"] / HBM_PEAK_GBPS, 4),
        "fused_call_frac_of_peak": round(head["fused_call_frac_of_peak"], 4),
        "worst_fused_call_frac_of_peak": round(min(v["fused_call_frac_of_peak"]
                                                   for v in results.values()), 4),
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_par,
        "copy_ceiling": copy_ceiling,
        "configs": configs,
        "context_parallel": cp,
        "tensor_parallel": tp,
        "decode_attention": dec,
        "host_allocator": host_alloc,
        "variants": {k_: {kk: (round(vv, 6) if isinstance(vv, float) else vv)
                          for kk, vv in v.items()} for k_, v in results.items()},
    }
    print(json.dumps(line), flush=True)


DECODE_Q_HEADS = 32  # Llama-3-8B attention: 32 query heads over the 8 key/value heads


def decode_bytes(w, ctx, num_q_heads, mode):
    """Algorithmic bytes of one decode-attention call: every readable position's K and V rows
    for all key/value heads, the queries read and the fp32 outputs written, and the mapping
    entries the positions resolve through (4 B per block-table entry in use; 12 B per range
    descriptor in use plus the count).  The chunk workspace is not counted."""
    import numpy as np
    kv = int(ctx.sum()) * w.num_kv_heads * w.head_dim * 2 * 2
    qo = w.num_reqs * num_q_heads * w.head_dim * (2 + 4)
    if mode == "paged":
        mapping = 4 * int(np.minimum(-(-ctx // w.block_size), w.num_blocks_per_req).sum())
    else:
        mapping = 12 * int(w.num_ranges.sum()) + 4 * w.num_reqs
    return kv + qo + mapping


def settle(fn, seconds=0.5):
    """Untimed calls of fn for at least `seconds` of GPU time."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def decode_attention(args, d, dev, stream, timed, planes=None):
    """Decode attention (one query per request) over the same cache layouts, paged gather vs
    range arithmetic: the 128K-context batch (16 requests) at 1 and 4096 ranges per request,
    and the 256-request decode step.  Time per call (both launches) from HIP events.

    planes: the write benchmark's K and V cache planes ([2, rows, row] int16), when there is
    one: the decode then reads views of them, allocated once at start-up as a serving cache
    is.  (A cache allocated after the write benchmark's large buffers were freed ran the same
    calls about 4% slower; the decode-only run allocates its own at start-up.)"""
    import numpy as np
    import torch

    import paged_kv_cache_46_amd as kvw
    from workloads import config, decode_inputs, long_context

    out = {}
    for wname, wl in (("long_context_r1", lambda: long_context(1)),
                      ("long_context_r4096", lambda: long_context(4096)),
                      ("decode_step", lambda: config("decode_step"))):
        w = wl()
        hq = DECODE_Q_HEADS
        q, ctx, _, _, _ = decode_inputs(w, hq, 77, rows=np.zeros(0, np.int64))
        ctx = ctx.astype(np.int64)
        max_ctx = int(ctx.max())
        rows = w.num_blocks * w.block_size
        n_elems = rows * w.num_kv_heads * w.head_dim
        if planes is not None and planes[0].numel() >= n_elems:
            kc = planes[0].reshape(-1)[:n_elems].view(rows, w.num_kv_heads, w.head_dim)
            vc = planes[1].reshape(-1)[:n_elems].view(rows, w.num_kv_heads, w.head_dim)
        else:
            kc = torch.empty((rows, w.num_kv_heads, w.head_dim), dtype=torch.int16, device=dev)
            vc = torch.empty_like(kc)
        # random bf16 payload drawn on the device (timing only; values do not change the work)
        for t in (kc, vc):
            t.view(torch.bfloat16).normal_()
        qd = d(q)
        cl = d(ctx.astype(np.int32))
        o = torch.empty((w.num_reqs, hq, w.head_dim), dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, kvw.kvw_decode_workspace_size(w.num_reqs, max_ctx, hq)),
                         dtype=torch.uint8, device=dev)
        maps = {"paged": dict(mode=kvw.KVW_SLOTS_PAGED, block_table=d(w.block_table),
                              num_blocks_per_req=d(w.num_blocks_per_req)),
                "ranges": dict(mode=kvw.KVW_SLOTS_RANGES, range_start=d(w.range_start),
                               range_len=d(w.range_len), range_cum=d(w.range_cum),
                               num_ranges=d(w.num_ranges))}
        # Right after the previous workload's caches are freed and these allocated, the same
        # call ran about 4% slower for its first ~0.2 s (measured on the decode step); the
        # workload's first timed configuration would carry that.  Untimed calls settle it.
        settle(lambda: kvw.kvw_decode_attention(q=qd, k_cache=kc, v_cache=vc, context_lens=cl,
                                                max_context=max_ctx, num_blocks=w.num_blocks,
                                                block_size=w.block_size, out=o, workspace=ws,
                                                **maps["paged"]))
        for mode, mp in maps.items():
            nbytes = decode_bytes(w, ctx, hq, mode)
            key = f"{wname}_{mode}"
            by_chunk = {}
            for chunk in (0, 256, 512, 1024, 2048):  # 0: the library's own choice, reported first
                def call(ev, mp=mp, chunk=chunk):
                    if ev is not None:
                        ev[0].record(stream)
                    kvw.kvw_decode_attention(q=qd, k_cache=kc, v_cache=vc, context_lens=cl,
                                             max_context=max_ctx, num_blocks=w.num_blocks,
                                             block_size=w.block_size, out=o, workspace=ws,
                                             chunk_positions=chunk, **mp)
                    if ev is not None:
                        ev[1].record(stream)
                wall, ev_ms = timed(call, args.warmup, args.steps)
                avg = statistics.fmean(ev_ms)
                by_chunk[chunk] = (avg, wall)
                log(f"[bench] decode attention {key:26s} chunk {chunk or 'auto':>4} "
                    f"{avg * 1e3:8.1f} us = {nbytes / (avg * 1e-3) / 1e9:5.0f} GB/s "
                    f"({100 * nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS:.1f}%)")
                del call
            avg, wall = by_chunk[0]
            out[key] = {"requests": w.num_reqs, "positions": int(ctx.sum()),
                        "max_context": max_ctx, "q_heads": hq, "kv_heads": w.num_kv_heads,
                        "block_size": w.block_size, "call_ms_avg": round(avg, 5),
                        "call_ms_wall": round(wall, 5), "algorithmic_bytes": nbytes,
                        "gbps": round(nbytes / (avg * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                        "call_ms_by_chunk": {str(c): round(v[0], 5) for c, v in by_chunk.items()
                                             if c}}
        if wname == "long_context_r1":
            for hq_g in (8, 16, 64):  # G = 1, 2 (the vector kernel) and 8 query heads per KV head
                out[f"long_context_r1_paged_g{hq_g // w.num_kv_heads}"] = decode_heads(
                    args, w, ctx, kc, vc, maps["paged"], d, timed, stream, kvw, torch, hq_g)
        if wname == "long_context_r4096":
            out["context_parallel_W2"] = decode_context_parallel(
                args, w, ctx, qd, cl, kc, vc, ws, maps["paged"], hq, timed, stream, kvw, torch)
        del kc, vc, ws
        torch.cuda.empty_cache()
    return out


def decode_heads(args, w, ctx, kc, vc, paged, d, timed, stream, kvw, torch, hq):
    """The 128K batch with hq query heads over the same 8 key/value heads (8 or 16: one or two
    per key/value head, the vector kernel; 64: eight, a 70B-class attention shape), paged, at
    the library's own chunk length."""
    import numpy as np

    from workloads import decode_inputs

    q = decode_inputs(w, hq, 78, rows=np.zeros(0, np.int64))[0]
    qd = d(q)
    cl = d(ctx.astype(np.int32))
    max_ctx = int(ctx.max())
    o = torch.empty((w.num_reqs, hq, w.head_dim), dtype=torch.float32, device=kc.device)
    ws = torch.empty(kvw.kvw_decode_workspace_size(w.num_reqs, max_ctx, hq), dtype=torch.uint8,
                     device=kc.device)

    def call(ev):
        if ev is not None:
            ev[0].record(stream)
        kvw.kvw_decode_attention(q=qd, k_cache=kc, v_cache=vc, context_lens=cl,
                                 max_context=max_ctx, num_blocks=w.num_blocks,
                                 block_size=w.block_size, out=o, workspace=ws, **paged)
        if ev is not None:
            ev[1].record(stream)
    wall, ev_ms = timed(call, args.warmup, args.steps)
    avg = statistics.fmean(ev_ms)
    nbytes = decode_bytes(w, ctx, hq, "paged")
    log(f"[bench] decode attention long_context_r1_paged G={hq // w.num_kv_heads}     {avg * 1e3:8.1f} us = "
        f"{nbytes / (avg * 1e-3) / 1e9:5.0f} GB/s "
        f"({100 * nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS:.1f}%)")
    return {"q_heads": hq, "kv_heads": w.num_kv_heads, "call_ms_avg": round(avg, 5),
            "call_ms_wall": round(wall, 5), "algorithmic_bytes": nbytes,
            "gbps": round(nbytes / (avg * 1e-3) / 1e9, 1),
            "frac_of_peak": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}


def decode_context_parallel(args, w, ctx, qd, cl, kc, vc, ws, paged, hq, timed, stream, kvw, torch):
    """Decode context parallelism at W = 2, interleave 1, paged: each rank attends the half of
    the positions it holds (timed one rank after the other on this GPU, each from a cache of
    block_size slots per block), then the ranks' results are merged by their log-sum-exp."""
    world = 2
    max_ctx = int(ctx.max())
    outs = torch.empty((world, w.num_reqs, hq, w.head_dim), dtype=torch.float32, device=kc.device)
    lses = torch.empty((world, w.num_reqs, hq), dtype=torch.float32, device=kc.device)
    res = {}
    for rank in range(world):
        def call(ev, rank=rank):
            if ev is not None:
                ev[0].record(stream)
            kvw.kvw_decode_attention(q=qd, k_cache=kc, v_cache=vc, context_lens=cl,
                                     max_context=max_ctx, num_blocks=w.num_blocks,
                                     block_size=w.block_size, out=outs[rank], workspace=ws,
                                     cp_world_size=world, cp_rank=rank, cp_interleave_size=1,
                                     lse_out=lses[rank], **paged)
            if ev is not None:
                ev[1].record(stream)
        _, ev_ms = timed(call, args.warmup, args.steps)
        avg = statistics.fmean(ev_ms)
        held = int(ctx.sum()) // world
        nbytes = held * w.num_kv_heads * w.head_dim * 2 * 2 + w.num_reqs * hq * w.head_dim * 6
        res[f"rank{rank}"] = {"positions": held, "call_ms_avg": round(avg, 5),
                              "gbps": round(nbytes / (avg * 1e-3) / 1e9, 1),
                              "frac_of_peak": round(nbytes / (avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        log(f"[bench] decode attention context parallel W=2 rank {rank}: {avg * 1e3:8.1f} us = "
            f"{res[f'rank{rank}']['gbps']:5.0f} GB/s")
    merged = torch.empty((w.num_reqs, hq, w.head_dim), dtype=torch.float32, device=kc.device)

    def merge(ev):
        if ev is not None:
            ev[0].record(stream)
        kvw.kvw_decode_merge(outs, lses, merged)
        if ev is not None:
            ev[1].record(stream)
    _, ev_ms = timed(merge, args.warmup, args.steps)
    res["merge_ms_avg"] = round(statistics.fmean(ev_ms), 5)
    log(f"[bench] decode attention context parallel W=2 merge: {res['merge_ms_avg'] * 1e3:.1f} us")
    return res


STUDY_CONFIGS = ("tiny_prefill", "decode_step", "mixed_chunked", "full_32_layer")
GRAPH_CONFIGS = ("tiny_prefill", "decode_step")  # launch-bound: also timed as graph replays


def config_results(name, steps, warmup, graph=False):
    """The fused write (paged, ranges) on one of the study configs other than the 128K one.

    Per variant: the fused call under the automatic schedule, the two-kernel and one-kernel
    schedules forced, and the slot mapping alone, each timed with HIP events after a 512 MiB
    write that evicts L2 and MALL; with `graph`, also the automatic call captured once in a HIP
    graph and replayed back to back (the pages run this path under graph replay, with a padded
    tail).  The K/V payload is seeded N(0, 1) bf16 drawn on the device: its values do not change
    the work, and the configs' host generator would take a minute for the 32-layer one."""
    import numpy as np
    import torch

    import paged_kv_cache_46_amd as kvw
    from workloads import BF16_SENTINEL, config

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def d(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    w = config(name)
    L, M, H, D = w.num_layers, w.max_num_tokens, w.num_kv_heads, w.head_dim
    log(f"[bench] workload {w.describe()}")
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    key = torch.randn((L, M, H, D), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    value = torch.randn((L, M, H, D), generator=gen, device=dev).to(torch.bfloat16).view(torch.int16)
    rows = L * w.num_blocks * w.block_size
    cache = torch.full((2, rows, H * D), BF16_SENTINEL, dtype=torch.int16, device=dev)
    sm_out = torch.empty(M, dtype=torch.int64, device=dev)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)  # evicts L2 and MALL
    qsl, pos = d(w.query_start_loc), d(w.positions)
    maps = {
        "paged": (kvw.KVW_SLOTS_PAGED, dict(block_table=d(w.block_table),
                                            num_blocks_per_req=d(w.num_blocks_per_req))),
        "ranges": (kvw.KVW_SLOTS_RANGES, dict(range_start=d(w.range_start),
                                              range_len=d(w.range_len), range_cum=d(w.range_cum),
                                              num_ranges=d(w.num_ranges))),
    }
    real = w.num_tokens
    fused_bytes = real * L * 4 * w.bytes_per_token + real * 16

    def flushed(call):
        for _ in range(warmup):
            call()
        times = []
        for i in range(steps):
            scratch.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        return times

    def entry(times):
        ms = statistics.fmean(times)
        return {"ms_avg": ms, "ms_p10": float(np.percentile(times, 10)),
                "ms_p90": float(np.percentile(times, 90)), "tokens_per_s": real / (ms * 1e-3),
                "gbps": fused_bytes / (ms * 1e-3) / 1e9,
                "frac_of_peak": fused_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}

    results = {}
    schedules = (("", kvw.KVW_SCHEDULE_AUTO), ("_two_kernels", kvw.KVW_SCHEDULE_TWO_KERNELS),
                 ("_one_kernel", kvw.KVW_SCHEDULE_ONE_KERNEL))
    for vname, (mode, mapping) in maps.items():
        for suffix, schedule in schedules:
            def call(mode=mode, mapping=mapping, schedule=schedule):
                kvw.kvw_kv_write(mode=mode, key=key, value=value, k_cache=cache[0],
                                 v_cache=cache[1], num_blocks=w.num_blocks,
                                 block_size=w.block_size, query_start_loc=qsl,
                                 num_reqs=w.num_reqs, positions=pos, slot_mapping_out=sm_out,
                                 schedule=schedule, **mapping)
            r = results[vname + suffix] = entry(flushed(call))
            log(f"[bench] {w.name} {vname + suffix:20s} {r['ms_avg'] * 1e3:8.1f} us  "
                f"{r['gbps']:6.0f} GB/s ({100 * r['frac_of_peak']:.1f}%)  "
                f"{r['tokens_per_s'] / 1e6:.2f} M tokens/s")
            if graph and not suffix:
                # `steps` calls captured in one HIP graph, as the write runs inside a replayed
                # model step: per-call GPU time with the calls back to back (a graph of one call
                # costs more host time per replay than the kernel runs)
                g = torch.cuda.CUDAGraph()
                side = torch.cuda.Stream()
                side.wait_stream(stream)
                with torch.cuda.stream(side):
                    call()
                stream.wait_stream(side)
                with torch.cuda.graph(g):
                    for _ in range(steps):
                        call()
                g.replay()
                reps = 5
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(reps):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / (reps * steps)
                results[vname + "_graph_replay"] = {
                    "ms_avg": ms, "tokens_per_s": real / (ms * 1e-3),
                    "gbps": fused_bytes / (ms * 1e-3) / 1e9,
                    "frac_of_peak": fused_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                    "timing": (f"{steps} calls captured in one graph, replayed {reps} times; per call, "
                               "no flush between calls")}
                log(f"[bench] {w.name} {vname + '_graph_replay':20s} {ms * 1e3:8.1f} us per call")
                del g
    for vname, (mode, mapping) in maps.items():  # the slot mapping alone (latency-bound)
        def smap(vname=vname, mapping=mapping):
            if vname == "paged":
                kvw.kvw_slot_mapping_paged(qsl, w.num_reqs, pos, M, mapping["block_table"],
                                           mapping["num_blocks_per_req"], w.block_size, sm_out)
            else:
                kvw.kvw_slot_mapping_ranges(qsl, w.num_reqs, pos, M, mapping["range_start"],
                                            mapping["range_len"], mapping["range_cum"],
                                            mapping["num_ranges"], w.block_size, sm_out)
        ms = statistics.fmean(flushed(smap))
        results[f"slot_mapping_{vname}"] = {"ms_avg": ms, "tokens_per_s": real / (ms * 1e-3)}
        log(f"[bench] {w.name} slot_mapping_{vname:8s} {ms * 1e3:8.1f} us  "
            f"{real / (ms * 1e-3) / 1e6:.1f} M tokens/s")
    del cache, key, value, scratch
    torch.cuda.empty_cache()
    return {"workload": w.name, "requests": w.num_reqs, "tokens_per_step": real,
            "max_num_tokens": M, "layers": L, "block_size": w.block_size,
            "num_blocks": w.num_blocks, "algorithmic_bytes_per_call": fused_bytes,
            "timing": "HIP events per call after a 512 MiB write evicting L2 and MALL",
            "variants": {k_: {kk: (round(vv, 6) if isinstance(vv, float) else vv)
                              for kk, vv in v.items()} for k_, v in results.items()}}


def slot_mapping_only():
    """The slot mapping alone, for hardware-counter runs: per layout, 10 paged then 10 range
    calls, each after a 512 MiB write that evicts L2 and MALL (so every call fetches its
    metadata from HBM).  Layouts in order: the 128K batch at R = 1, 16, 512, 4096 (manager
    block size 32: the write's own mapping), the decode step, the mixed batch.  Returns the
    order of the calls."""
    import numpy as np
    import torch

    import paged_kv_cache_46_amd as kvw
    from workloads import config, long_context

    dev = torch.device("cuda:0")

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    order = []
    layouts = [(f"long_context_r{r}", lambda r=r: long_context(r)) for r in (1, 16, 512, 4096)]
    layouts += [(n, lambda n=n: config(n)) for n in ("decode_step", "mixed_chunked")]
    for name, make in layouts:
        w = make()
        qsl, pos = d(w.query_start_loc), d(w.positions)
        bt, nb = d(w.block_table), d(w.num_blocks_per_req)
        rs, rl, rc, nr = (d(a) for a in (w.range_start, w.range_len, w.range_cum, w.num_ranges))
        sm = torch.empty(w.max_num_tokens, dtype=torch.int64, device=dev)
        for variant in ("paged", "ranges"):
            for i in range(10):
                scratch.fill_(i)
                if variant == "paged":
                    kvw.kvw_slot_mapping_paged(qsl, w.num_reqs, pos, w.max_num_tokens, bt, nb,
                                               w.block_size, sm)
                else:
                    kvw.kvw_slot_mapping_ranges(qsl, w.num_reqs, pos, w.max_num_tokens, rs, rl, rc,
                                                nr, w.block_size, sm)
            torch.cuda.synchronize()
            order.append({"layout": name, "variant": variant, "calls": 10,
                          "tokens": w.num_tokens, "requests": w.num_reqs,
                          "runs": int(w.num_ranges[:w.num_reqs].sum())})
            log(f"[bench] slot mapping {name} {variant}: 10 calls")
    return {"slot_mapping_calls": order}


def bench_config(args):
    """One JSON line for one of the other study configs (--workload)."""
    res = config_results(args.workload, args.steps, args.warmup,
                         graph=args.workload in GRAPH_CONFIGS)
    head = res["variants"]["paged"]
    line = {
        "metric": METRIC, "value": round(head["tokens_per_s"], 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(head["ms_avg"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int64", "data": "synthetic",
        "config": {"workload": res["workload"], "requests": res["requests"],
                   "tokens_per_step": res["tokens_per_step"], "max_num_tokens": res["max_num_tokens"],
                   "layers": res["layers"], "block_size": res["block_size"],
                   "num_blocks": res["num_blocks"], "kv_heads": 8, "head_dim": 128,
                   "payload": "bf16", "variant": "paged",
                   "timing": "fused call, HIP events, L2/MALL flushed"},
        "hbm_gbps": round(head["gbps"], 1), "hbm_frac_of_peak": round(head["frac_of_peak"], 4),
        "algorithmic_bytes_per_step": res["algorithmic_bytes_per_call"],
        "variants": res["variants"],
    }
    print(json.dumps(line), flush=True)


# Host figures of the same scenarios published on "Range-addressed KV cache blocks for the vLLM
# serving engine" ("Measured Results"), measured there on an Apple arm64 host: context, not a target.
PUBLISHED_HOST_NS = {"map/offset single": 1.85, "map/offset decode walk": 1.85,
                     "map/offset context walk 4k": 1.71, "alloc/allocate release": 66.6,
                     "alloc/grow in place": 25.8, "alloc/prefix acquire release": 4.3,
                     "alloc/evict cache only": 71.6}


def host_allocator():
    """Run the native host benchmark of the range allocator (paged_kv_cache_46_amd/bench_alloc)."""
    import platform
    import subprocess

    from paged_kv_cache_46_amd.build import BENCH_ALLOC
    if not os.path.exists(BENCH_ALLOC):
        log("[bench] bench_alloc not built; host allocator figures skipped")
        return None
    r = subprocess.run([BENCH_ALLOC, "200000", "20"], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        log(f"[bench] bench_alloc failed: {r.stderr[-500:]}")
        return None
    out = {}
    for ln in r.stdout.splitlines():
        d = json.loads(ln)
        name = d.pop("scenario")
        d["published_ns"] = PUBLISHED_HOST_NS.get(name)
        out[name] = d
        log(f"[bench] host {name:30s} {d['mean_ns']:8.2f} +- {d['stddev_ns']:.2f} {d['unit']}"
            f"  (published {d['published_ns']})")
    cpu = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                if ln.startswith("model name")), platform.processor())
    return {"cpu": cpu, "harness": "iterations x rounds, one warmup call per round, steady clock",
            "scenarios": out}


def cpu_baseline(w, budget_s):
    """The CPU oracle on the same 128K batch (paged chain), harness of iterations x rounds
    with one warmup call per round; single-threaded."""
    import numpy as np

    import oracle

    orc = oracle.get()
    key = w.kv_layer(0, 0)[None]
    value = w.kv_layer(1, 0)[None]
    k = w.blocks_per_kv_block
    rows = w.kernel_num_blocks * w.kernel_block_size
    kwin = np.empty((rows, w.row_elems), np.uint16)  # touched lazily: only written rows page in
    vwin = np.empty_like(kwin)

    def call():
        kt, _ = orc.map_to_kernel_blocks(w.block_table, w.num_blocks_per_req, w.block_size,
                                         w.kernel_block_size)
        sm, _ = orc.slot_mapping_paged(w.query_start_loc, w.num_reqs, w.positions,
                                       w.max_num_tokens, kt, w.num_blocks_per_req * k,
                                       w.kernel_block_size)
        orc.kv_write(sm, key, value, w.kernel_num_blocks, w.kernel_block_size, kwin, vwin)

    call()  # first touch of the written pages
    t = time.perf_counter()
    call()
    one = time.perf_counter() - t
    rounds = 5
    iters = max(1, int(budget_s / rounds / max(one, 1e-6)))
    per_call = []
    for _ in range(rounds):
        call()  # warmup call of the round
        t = time.perf_counter()
        for _ in range(iters):
            call()
        per_call.append((time.perf_counter() - t) / iters)
    mean = statistics.fmean(per_call)
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    res = {
        "value": round(w.num_tokens / mean, 1),
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"the whole 128K batch ({w.num_tokens} tokens), paged chain: expansion + "
                   f"slot mapping + K/V write into host cache planes; {rounds} rounds x {iters} "
                   "calls, one warmup call per round"),
        "ms_per_call_mean": round(mean * 1e3, 3),
        "ms_per_call_std": round(statistics.pstdev(per_call) * 1e3, 3),
        "host_cpu": model,
        "host_logical_cpus": os.cpu_count(),
    }
    log(f"[bench] CPU oracle: {mean * 1e3:.1f} ms per batch = {res['value'] / 1e6:.2f} M tokens/s "
        f"(1 thread, {model})")
    return res


def cpu_baseline_threads(w, budget_s, max_threads=16):
    """The same oracle chain with the batch's requests split over threads (at most 16, the
    host share of one GPU): thread i runs the unchanged oracle calls on its own requests, whose
    tokens and cache rows are disjoint from the others'.  The oracle's C calls release the
    interpreter lock, so the threads run in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    orc = oracle.get()
    key = w.kv_layer(0, 0)[None]
    value = w.kv_layer(1, 0)[None]
    k = w.blocks_per_kv_block
    rows = w.kernel_num_blocks * w.kernel_block_size
    kwin = np.empty((rows, w.row_elems), np.uint16)
    vwin = np.empty_like(kwin)
    threads = max(1, min(max_threads, os.cpu_count() or 1, w.num_reqs))
    bounds = np.linspace(0, w.num_reqs, threads + 1).astype(int)
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        t0, t1 = int(w.query_start_loc[a]), int(w.query_start_loc[b])
        parts.append(dict(qsl=np.ascontiguousarray(w.query_start_loc[a:b + 1] - t0),
                          nreq=int(b - a), pos=np.ascontiguousarray(w.positions[t0:t1]),
                          table=np.ascontiguousarray(w.block_table[a:b]),
                          nbpr=np.ascontiguousarray(w.num_blocks_per_req[a:b]),
                          key=np.ascontiguousarray(key[:, t0:t1]),
                          value=np.ascontiguousarray(value[:, t0:t1])))

    def run(pt):
        kt, _ = orc.map_to_kernel_blocks(pt["table"], pt["nbpr"], w.block_size,
                                         w.kernel_block_size)
        sm, _ = orc.slot_mapping_paged(pt["qsl"], pt["nreq"], pt["pos"], len(pt["pos"]), kt,
                                       pt["nbpr"] * k, w.kernel_block_size)
        orc.kv_write(sm, pt["key"], pt["value"], w.kernel_num_blocks, w.kernel_block_size, kwin,
                     vwin)

    with ThreadPoolExecutor(threads) as ex:
        def call():
            list(ex.map(run, parts))
        call()  # first touch of the written pages
        t = time.perf_counter()
        call()
        one = time.perf_counter() - t
        rounds = 5
        iters = max(1, int(budget_s / rounds / max(one, 1e-6)))
        per_call = []
        for _ in range(rounds):
            call()
            t = time.perf_counter()
            for _ in range(iters):
                call()
            per_call.append((time.perf_counter() - t) / iters)
    mean = statistics.fmean(per_call)
    res = {"value": round(w.num_tokens / mean, 1), "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": (f"the whole 128K batch, its {w.num_reqs} requests split over {threads} "
                      f"threads; {rounds} rounds x {iters} calls, one warmup call per round"),
           "ms_per_call_mean": round(mean * 1e3, 3),
           "ms_per_call_std": round(statistics.pstdev(per_call) * 1e3, 3)}
    log(f"[bench] CPU oracle, {threads} threads: {mean * 1e3:.1f} ms per batch = "
        f"{res['value'] / 1e6:.2f} M tokens/s")
    return res


if __name__ == "__main__":
    main()
