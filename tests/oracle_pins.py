"""Checks that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:
  * values the pages print (fixtures under tests/golden/, each cited there);
  * a token-at-a-time allocation simulation that places every token by
    counting free slots (no division, no modulo, no table lookup);
  * enumeration of every slot a request owns, in logical order;
  * the pages' invariant that range arithmetic and the table gather give the
    same slot for the same physical layout, and that a table filled from the
    runs is the runs laid end to end;
  * a dealing simulation (no division) of the context-parallel placement;
  * closed forms of decode attention (one token, zero query, the two-token logistic
    weights, a dominant score, constant value rows per head, linearity, placement);
  * numpy's own row-major indexing (ravel_multi_index, array addresses,
    fancy-index scatter) for the coordinate form and the K/V copy.
The same functions are run against deliberately broken builds of the oracle
(test_oracle_mutants.py) to show that each plausible mistake is caught.
"""
from __future__ import annotations

import os
from typing import Dict, List, Tuple

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
PAD = -1


# ---------------------------------------------------------------------------
# fixture parsing
# ---------------------------------------------------------------------------
def _lines(name: str) -> List[List[str]]:
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                out.append(ln.split())
    return out


def _runs_of(row: List[int]) -> List[Tuple[int, int, int]]:
    """Compress a block row into maximal runs of consecutive ids: (start, len, cum)."""
    runs: List[Tuple[int, int, int]] = []
    for j, b in enumerate(row):
        if runs and runs[-1][0] + runs[-1][1] == b:
            s, ln, c = runs[-1]
            runs[-1] = (s, ln + 1, c)
        else:
            runs.append((b, 1, j))
    return runs


def _descriptors(rows: List[List[int]], stride: int = 0):
    runs = [_runs_of(r) for r in rows]
    stride = max(stride, max((len(r) for r in runs), default=1), 1)
    R = len(rows)
    st, ln, cm = (np.zeros((R, stride), np.int32) for _ in range(3))
    nr = np.zeros(R, np.int32)
    for i, rr in enumerate(runs):
        nr[i] = len(rr)
        for k, (s, l, c) in enumerate(rr):
            st[i, k], ln[i, k], cm[i, k] = s, l, c
    return st, ln, cm, nr


def _table(rows: List[List[int]], stride: int = 0):
    stride = max(stride, max((len(r) for r in rows), default=1), 1)
    t = np.zeros((len(rows), stride), np.int32)
    for i, r in enumerate(rows):
        t[i, :len(r)] = r
    return t, np.array([len(r) for r in rows], np.int32)


def _batch(scheduled: List[List[int]], pad_to: int = 0, rng=None):
    """qsl and positions for requests scheduling the given positions (in order)."""
    counts = [len(s) for s in scheduled]
    qsl = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(qsl[-1])
    m = max(n, pad_to)
    pos = np.empty(m, np.int64)
    pos[:n] = [p for s in scheduled for p in s]
    if m > n:
        g = rng if rng is not None else np.random.default_rng(0)
        pos[n:] = g.integers(-(1 << 20), 1 << 20, size=m - n)
    return qsl, pos, m


def _both(orc, qsl, pos, m, rows, bs, table_stride=0):
    t, nb = _table(rows, table_stride)
    st, ln, cm, nr = _descriptors(rows)
    paged, fp = orc.slot_mapping_paged(qsl, len(rows), pos, m, t, nb, bs)
    ranges, fr = orc.slot_mapping_ranges(qsl, len(rows), pos, m, st, ln, cm, nr, bs)
    return paged, ranges, fp, fr


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------
def pin_golden_bs16(orc):
    """Printed slot values for row [7, 1] at block size 16."""
    bs, row, slots, spans = None, None, {}, []
    for f in _lines("slot_mapping_bs16.txt"):
        if f[0] == "block_size":
            bs = int(f[1])
        elif f[0] == "row":
            row = [int(x) for x in f[1:]]
        elif f[0] == "slot":
            slots[int(f[1])] = int(f[2])
        elif f[0] == "block":
            spans.append((int(f[1]), int(f[2]), int(f[3])))
    last = max(b for _, b, _ in spans)
    qsl, pos, m = _batch([list(range(0, last + 1))])
    paged, ranges, _, _ = _both(orc, qsl, pos, m, [row], bs)
    for out in (paged, ranges):
        for p, s in slots.items():
            assert out[p] == s, (p, out[p], s)
        for a, b, blk in spans:
            for p in range(a, b + 1):
                assert blk * bs <= out[p] < (blk + 1) * bs, (p, out[p], blk)
        assert len(set(out.tolist())) == len(out)


def pin_figure6(orc):
    """Figure 6 sequence: prompt into blocks 7 and 1, decode into the free slot, then block 3."""
    bs, steps = None, []
    for f in _lines("figure6_bs4.txt"):
        if f[0] == "block_size":
            bs = int(f[1])
        elif f[0] == "step":
            steps.append(([int(x) for x in f[2:]], []))
        elif f[0] == "place":
            steps[-1][1].append((int(f[1]), int(f[2]), int(f[3])))
    for row, places in steps:
        qsl, pos, m = _batch([[p for p, _, _ in places]], pad_to=len(places) + 3)
        paged, ranges, _, _ = _both(orc, qsl, pos, m, [row], bs)
        for out in (paged, ranges):
            for i, (p, blk, idx) in enumerate(places):
                assert out[i] == blk * bs + idx, (row, p, out[i], blk, idx)
            assert (out[len(places):] == PAD).all()


def _simulate(rng, lengths: List[int], bs: int, pool: int, run_free_list: bool):
    """Place tokens one at a time; a request takes a fresh block when its last one is full.

    Returns rows (physical blocks in logical order) and, per request, the
    (block, index-in-block) of every position.  With run_free_list the free
    list hands out shuffled runs of consecutive ids (so rows compress into
    ranges); otherwise single ids in random order.
    """
    ids = list(range(1, pool))
    if run_free_list:
        runs, i = [], 0
        while i < len(ids):
            ln = int(rng.integers(1, 6))
            runs.append(ids[i:i + ln])
            i += ln
        order = rng.permutation(len(runs))
        free = [b for k in order for b in runs[k]]
    else:
        free = [ids[k] for k in rng.permutation(len(ids))]
    free.reverse()  # pop() from the end == take from the head
    rows, places = [], []
    # interleave requests token by token, as continuous batching would
    fill = [bs] * len(lengths)
    rows = [[] for _ in lengths]
    places = [[] for _ in lengths]
    left = list(lengths)
    while any(left):
        for r in range(len(lengths)):
            if not left[r]:
                continue
            if fill[r] == bs:
                rows[r].append(free.pop())
                fill[r] = 0
            places[r].append((rows[r][-1], fill[r]))
            fill[r] += 1
            left[r] -= 1
    return rows, places


def pin_fill_simulation(orc, seeds=range(6)):
    """Slots agree with a token-at-a-time placement for random batches."""
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)
        bs = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        n_req = int(rng.integers(1, 6))
        lengths = [int(rng.integers(1, 70)) for _ in range(n_req)]
        need = sum(-(-ln // bs) for ln in lengths)
        rows, places = _simulate(rng, lengths, bs, need + 40, run_free_list=bool(seed % 2))
        # each request schedules its last n_new positions this step
        sched, expect = [], []
        for ln, plc in zip(lengths, places):
            n_new = int(rng.integers(0, ln + 1))
            sched.append(list(range(ln - n_new, ln)))
            expect += [b * bs + i for (b, i) in plc[ln - n_new:]]
        qsl, pos, m = _batch(sched, pad_to=len(expect) + int(rng.integers(0, 9)), rng=rng)
        paged, ranges, _, _ = _both(orc, qsl, pos, m, rows, bs,
                                    table_stride=int(rng.integers(0, 4)) + max(map(len, rows)))
        n = len(expect)
        for out in (paged, ranges):
            assert out[:n].tolist() == expect, (seed, out[:n].tolist(), expect)
            assert (out[n:] == PAD).all()


def pin_enumeration(orc):
    """Exhaustive tiny layouts: position p owns the p-th slot of the request, in logical order."""
    rng = np.random.default_rng(7)
    for bs in (1, 2, 3):
        for lens in ([1], [2], [1, 1], [2, 1], [1, 2, 1], [2, 2, 2]):
            for trial in range(3):
                starts = rng.choice(np.arange(1, 40, 3), size=len(lens), replace=False)
                row = [int(s) + j for s, ln in zip(starts, lens) for j in range(ln)]
                owned = [b * bs + i for b in row for i in range(bs)]
                positions = list(range(-2, len(owned) + bs + 1))
                qsl, pos, m = _batch([positions])
                paged, ranges, _, _ = _both(orc, qsl, pos, m, [row], bs)
                for out in (paged, ranges):
                    for i, p in enumerate(positions):
                        want = owned[p] if 0 <= p < len(owned) else PAD
                        assert out[i] == want, (bs, lens, p, out[i], want)


def pin_padding_rules(orc):
    """Tail, negative positions, unowned blocks, clamped counts and num_tokens."""
    bs = 4
    rows = [[5, 6], [9]]
    # request 0: positions 0..9 (blocks 0,1 owned, 2 not); request 1: -1, 3, 4
    sched = [list(range(10)), [-1, 3, 4]]
    qsl, pos, m = _batch(sched, pad_to=20)
    t, nb = _table(rows, 3)
    paged, f = orc.slot_mapping_paged(qsl, 2, pos, m, t, nb, bs)
    want = [20, 21, 22, 23, 24, 25, 26, 27, PAD, PAD, PAD, 39, PAD] + [PAD] * 7
    assert paged.tolist() == want, paged.tolist()
    assert f == 0
    # without per-row counts the whole row width is owned; unfilled entries are block 0
    paged, _ = orc.slot_mapping_paged(qsl, 2, pos, m, t, None, bs)
    assert paged[8] == 0 and paged[9] == 1 and paged[13] == PAD
    # counts beyond the row width are clamped and flagged
    paged, f = orc.slot_mapping_paged(qsl, 2, pos, m, t, np.array([9, 1], np.int32), bs)
    assert f & 2 and paged[8] == 0
    # num_tokens past max_num_tokens is clamped and flagged
    q2 = qsl.copy()
    q2[-1] = 25
    paged, f = orc.slot_mapping_paged(q2, 2, pos, m, t, nb, bs)
    assert f & 1 and paged[12] == PAD and paged[11] == 39
    # ranges: same layout, same rules
    st, ln, cm, nr = _descriptors(rows)
    ranges, f = orc.slot_mapping_ranges(qsl, 2, pos, m, st, ln, cm, nr, bs)
    assert ranges.tolist() == want
    # dummy requests with no tokens and no ranges contribute nothing
    qd = np.array([0, 3, 3, 3], np.int32)
    pd = np.array([0, 1, 2, 77, 78], np.int64)
    td, nbd = _table([[2], [], []], 2)
    out, _ = orc.slot_mapping_paged(qd, 3, pd, 5, td, nbd, bs)
    assert out.tolist() == [8, 9, 10, PAD, PAD]


def pin_range_equals_gather(orc, workloads):
    """The pages' invariant: range arithmetic == gather through the materialized table."""
    for w in workloads:
        paged, _ = orc.slot_mapping_paged(w.query_start_loc, w.num_reqs, w.positions,
                                          w.max_num_tokens, w.block_table, w.num_blocks_per_req,
                                          w.block_size)
        ranges, _ = orc.slot_mapping_ranges(w.query_start_loc, w.num_reqs, w.positions,
                                            w.max_num_tokens, w.range_start, w.range_len,
                                            w.range_cum, w.num_ranges, w.block_size)
        assert np.array_equal(paged, ranges), w.name
        n = w.num_tokens
        assert (paged[n:] == PAD).all()
        real = paged[:n][paged[:n] >= 0]
        assert len(np.unique(real)) == len(real), w.name


def pin_expansion(orc):
    """Manager->kernel expansion keeps every token's slot (same memory, finer blocks)."""
    rng = np.random.default_rng(11)
    for (bs_m, bs_k) in ((32, 16), (64, 16), (16, 16), (48, 16), (12, 4)):
        k = bs_m // bs_k
        lengths = [int(rng.integers(1, 200)) for _ in range(4)]
        need = sum(-(-ln // bs_m) for ln in lengths)
        rows, places = _simulate(rng, lengths, bs_m, need + 30, run_free_list=True)
        sched = [list(range(ln)) for ln in lengths]
        qsl, pos, m = _batch(sched, pad_to=sum(lengths) + 5)
        expect = [b * bs_m + i for plc in places for (b, i) in plc]
        t, nb = _table(rows, max(map(len, rows)) + 2)
        kt, kc, f = orc.map_to_kernel_blocks(t, nb, bs_m, bs_k, with_counts=True)
        assert f == 0 and kt.shape[1] == t.shape[1] * k
        assert kc.tolist() == [len(row) * k for row in rows]
        # row r, manager block i covers kernel blocks i*k .. i*k+k-1 of the same memory
        for r, row in enumerate(rows):
            for i, b in enumerate(row):
                for j in range(k):
                    assert kt[r, i * k + j] * bs_k == b * bs_m + j * bs_k
            assert (kt[r, len(row) * k:] == 0).all()
        sm, _ = orc.slot_mapping_paged(qsl, len(rows), pos, m, kt, nb * k, bs_k)
        assert sm[:len(expect)].tolist() == expect
        st, ln, cm, nr = _descriptors(rows)
        (ks, kl, kc, kn), f = orc.map_ranges_to_kernel_blocks(st, ln, cm, nr, bs_m, bs_k)
        assert f == 0 and np.array_equal(kn, nr)
        sr, _ = orc.slot_mapping_ranges(qsl, len(rows), pos, m, ks, kl, kc, kn, bs_k)
        assert sr[:len(expect)].tolist() == expect
        sr32, _ = orc.slot_mapping_ranges(qsl, len(rows), pos, m, st, ln, cm, nr, bs_m)
        assert np.array_equal(sr32, sr)
    # a kernel block size that does not divide the manager block size is rejected
    from oracle import OracleError
    for bad in ((32, 12), (16, 32), (16, 0)):
        try:
            orc.map_to_kernel_blocks(np.ones((1, 2), np.int32), None, *bad)
        except OracleError:
            pass
        else:
            raise AssertionError(f"expansion {bad} not rejected")


def pin_table_fill(orc, workloads=()):
    """Block table filled from range descriptors == the request's runs laid end to end.

    The printed rows ([7, 1] at block size 16, the Figure 6 rows) come back
    from their descriptors; rows of the token-at-a-time simulation round-trip
    through run compression (``_runs_of``, written independently above); at a
    finer kernel block size, entry q of a row names the same memory as manager
    block q // k; the filled table drives the gather to the slots the
    simulation placed; truncation, clamped counts and unrepresentable ids are
    flagged; and every generated workload's own table is reproduced.
    """
    from oracle import FLAG_BAD_BLOCK, FLAG_COUNT
    printed = [[int(x) for x in f[1:]] for f in _lines("slot_mapping_bs16.txt") if f[0] == "row"]
    printed += [[int(x) for x in f[2:]] for f in _lines("figure6_bs4.txt") if f[0] == "step"]
    assert [7, 1] in printed and [7, 1, 3] in printed
    for row in printed:
        st, ln, cm, nr = _descriptors([row])
        out, cnt, f = orc.ranges_to_block_table(st, ln, cm, nr, 1, 1, len(row) + 3)
        assert out[0].tolist() == row + [0, 0, 0] and cnt.tolist() == [len(row)] and f == 0, row

    rng = np.random.default_rng(23)
    for trial in range(12):
        bs_m, bs_k = [(16, 16), (32, 16), (64, 16), (12, 4), (4, 1), (3, 3)][trial % 6]
        k = bs_m // bs_k
        lengths = [int(rng.integers(1, 90)) for _ in range(int(rng.integers(1, 5)))]
        need = sum(-(-ln // bs_m) for ln in lengths)
        rows, places = _simulate(rng, lengths, bs_m, need + 30, run_free_list=trial % 2 == 0)
        st, ln, cm, nr = _descriptors(rows, stride=int(rng.integers(0, 3)))
        width = max(map(len, rows)) * k + int(rng.integers(0, 5))
        out, cnt, f = orc.ranges_to_block_table(st, ln, cm, nr, bs_m, bs_k, width)
        assert f == 0 and out.shape == (len(rows), width)
        for r, row in enumerate(rows):
            assert cnt[r] == len(row) * k
            for q in range(len(row) * k):
                assert out[r, q] * bs_k == row[q // k] * bs_m + (q % k) * bs_k, (trial, r, q)
            assert (out[r, len(row) * k:] == 0).all()
        qsl, pos, m = _batch([list(range(n)) for n in lengths], pad_to=sum(lengths) + 4, rng=rng)
        expect = [b * bs_m + i for plc in places for (b, i) in plc]
        sm, _ = orc.slot_mapping_paged(qsl, len(rows), pos, m, out, cnt, bs_k)
        assert sm[:len(expect)].tolist() == expect and (sm[len(expect):] == PAD).all(), trial

    # runs (5, 3) and (9, 2) at k = 2: ten kernel ids, of which a 4-wide row keeps four
    st, ln, cm, nr = _descriptors([[5, 6, 7, 9, 10]])
    out, cnt, f = orc.ranges_to_block_table(st, ln, cm, nr, 2, 1, 4)
    assert out.tolist() == [[10, 11, 12, 13]] and cnt.tolist() == [4] and f == FLAG_COUNT
    out, cnt, f = orc.ranges_to_block_table(st, ln, cm, nr, 2, 1, 12)
    assert out.tolist() == [[10, 11, 12, 13, 14, 15, 18, 19, 20, 21, 0, 0]] and cnt.tolist() == [10]
    assert f == 0
    # a count outside [0, range_stride] is clamped and flagged
    out, cnt, f = orc.ranges_to_block_table(st, ln, cm, np.array([7], np.int32), 1, 1, 6)
    assert out.tolist() == [[5, 6, 7, 9, 10, 0]] and cnt.tolist() == [5] and f == FLAG_COUNT
    out, cnt, f = orc.ranges_to_block_table(st, ln, cm, np.array([-1], np.int32), 1, 1, 3)
    assert out.tolist() == [[0, 0, 0]] and cnt.tolist() == [0] and f == FLAG_COUNT
    # negative ids and ids whose kernel id leaves int32 become the null block
    big = (1 << 31) // 2 - 1  # big*2 + 1 == INT32_MAX: representable; big + 1 is not
    st = np.array([[-3, big]], np.int32)
    ln = np.array([[2, 2]], np.int32)
    cm = np.array([[0, 2]], np.int32)
    out, cnt, f = orc.ranges_to_block_table(st, ln, cm, np.array([2], np.int32), 2, 1, 8)
    assert out.tolist() == [[0, 0, 0, 0, 2 * big, 2 * big + 1, 0, 0]] and cnt.tolist() == [8]
    assert f == FLAG_BAD_BLOCK

    for w in workloads:
        out, cnt, f = orc.ranges_to_block_table(w.range_start, w.range_len, w.range_cum,
                                                w.num_ranges, w.block_size, w.block_size,
                                                w.table_stride)
        assert f == 0 and np.array_equal(out, w.block_table), w.name
        assert np.array_equal(cnt, w.num_blocks_per_req), w.name


def _deal(rows: List[List[int]], lengths: List[int], bs: int, world: int, interleave: int):
    """Context parallelism by dealing, with no division: each request's positions are dealt to
    the ranks in turn, `interleave` at a time; a virtual block of bs*world positions is one
    table entry, and each rank takes the next free slot of its own copy of that block.
    Returns, per request, the (rank, slot) of every position (slot None past the row)."""
    out = []
    for row, n in zip(rows, lengths):
        placed = []
        rank, dealt, v, in_v = 0, 0, 0, 0
        fill = [0] * world
        for _ in range(n):
            if v < len(row):
                placed.append((rank, row[v] * bs + fill[rank]))
            else:
                placed.append((rank, None))
            fill[rank] += 1
            dealt += 1
            if dealt == interleave:
                dealt, rank = 0, (rank + 1) % world
            in_v += 1
            if in_v == bs * world:
                in_v, v, fill = 0, v + 1, [0] * world
        out.append(placed)
    return out


def pin_context_parallel(orc, workloads=()):
    """Context-parallel slot mapping (a reading: the pages name the parameters, not the layout).

    Each rank's slots equal a dealing simulation; over the ranks every position is held exactly
    once and every (rank, slot) is distinct; ranges and the gather agree on every rank; W = 1
    is the plain mapping for any interleave size; invalid parameters are rejected."""
    from oracle import OracleError
    rng = np.random.default_rng(31)
    for trial in range(16):
        bs = [4, 8, 16, 6, 2, 12][trial % 6]
        world = [2, 3, 4, 8][trial % 4]
        interleave = int(rng.choice([i for i in range(1, bs + 1) if bs % i == 0]))
        lengths = [int(rng.integers(1, 4 * bs * world)) for _ in range(int(rng.integers(1, 5)))]
        vbs = bs * world
        rows, _ = _simulate(rng, lengths, vbs, sum(-(-n // vbs) for n in lengths) + 20,
                            run_free_list=trial % 2 == 0)
        rows = [r[:len(r) - int(rng.integers(0, 2))] or r for r in rows]  # some rows end early
        dealt = _deal(rows, lengths, bs, world, interleave)
        sched, want = [], []
        for n, plc in zip(lengths, dealt):
            k = int(rng.integers(1, n + 1))
            sched.append(list(range(n - k, n)))
            want.append(plc[n - k:])
        qsl, pos, m = _batch(sched, pad_to=sum(map(len, sched)) + 3, rng=rng)
        t_, nb = _table(rows)
        st, ln, cm, nr = _descriptors(rows)
        seen = set()
        held = np.zeros(m, np.int64)
        for rank in range(world):
            paged, fp = orc.slot_mapping_paged_cp(qsl, len(rows), pos, m, t_, nb, bs, world, rank,
                                                  interleave)
            ranges, fr = orc.slot_mapping_ranges_cp(qsl, len(rows), pos, m, st, ln, cm, nr, bs,
                                                    world, rank, interleave)
            assert np.array_equal(paged, ranges) and fp == fr == 0, (trial, rank)
            flat = [x for plc in want for x in plc]
            for i, (owner, slot) in enumerate(flat):
                expect = slot if owner == rank and slot is not None else PAD
                assert paged[i] == expect, (trial, rank, i, paged[i], expect)
            assert (paged[len(flat):] == PAD).all()
            for i in np.nonzero(paged >= 0)[0]:
                assert (rank, int(paged[i])) not in seen
                seen.add((rank, int(paged[i])))
                held[i] += 1
        n_real = sum(1 for plc in want for (_, s) in plc if s is not None)
        assert held.sum() == n_real and held.max(initial=0) <= 1

    for w in workloads:
        plain, _ = orc.slot_mapping_paged(w.query_start_loc, w.num_reqs, w.positions,
                                          w.max_num_tokens, w.block_table, w.num_blocks_per_req,
                                          w.block_size)
        for interleave in [i for i in (1, 2, w.block_size) if w.block_size % i == 0]:
            cp, _ = orc.slot_mapping_paged_cp(w.query_start_loc, w.num_reqs, w.positions,
                                              w.max_num_tokens, w.block_table,
                                              w.num_blocks_per_req, w.block_size, 1, 0,
                                              interleave)
            assert np.array_equal(cp, plain), (w.name, interleave)
            cr, _ = orc.slot_mapping_ranges_cp(w.query_start_loc, w.num_reqs, w.positions,
                                               w.max_num_tokens, w.range_start, w.range_len,
                                               w.range_cum, w.num_ranges, w.block_size, 1, 0,
                                               interleave)
            assert np.array_equal(cr, plain), (w.name, interleave)

    qsl, pos, m = _batch([list(range(20))])
    t_, nb = _table([[3, 5]])
    for bad in ((16, 2, 2, 1), (16, 2, -1, 1), (16, 0, 0, 1), (16, 2, 0, 3), (16, 2, 0, 0),
                (16, 2, 0, 32)):
        try:
            orc.slot_mapping_paged_cp(qsl, 1, pos, m, t_, nb, *bad)
        except OracleError:
            continue
        raise AssertionError(f"context-parallel parameters {bad} not rejected")


def _bf16(x):
    """float -> bf16 bit pattern, rounding to nearest even (exact for the small integers and
    halves used below)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_attention(orc):
    """Decode attention: closed forms and invariants, none of them a restatement of the loops."""
    rng = np.random.default_rng(41)
    hq, hkv, d = 8, 2, 16
    group = hq // hkv
    rows = 40
    q = _bf16(rng.standard_normal((3, hq, d)))
    k = _bf16(rng.standard_normal((rows, hkv, d)))
    v = _bf16(rng.standard_normal((rows, hkv, d)))
    scale = 1.0 / np.sqrt(d)
    vv = _bf16_value(v)
    # one token: its value row, exactly, for every head
    out = orc.decode_attention(q, k, v, [[7]], [1], hq, hkv, scale)
    for h in range(hq):
        assert np.array_equal(out[0, h], vv[7, h // group])
    # no token: zeros
    assert not orc.decode_attention(q, k, v, [[]], [1], hq, hkv, scale).any()
    # zero query: uniform weights, the mean of the value rows
    qz = np.zeros_like(q)
    sl = [3, 9, 11, 20, 21, 33]
    out = orc.decode_attention(qz, k, v, [sl], [0], hq, hkv, scale)
    for h in range(hq):
        assert np.allclose(out[0, h], vv[sl, h // group].mean(axis=0), rtol=0, atol=1e-13)
    # two tokens with one-hot keys: weights are the logistic function of the score gap
    q2 = np.zeros_like(q)
    q2[:, :, 0] = _bf16(2.0)
    k2 = np.zeros_like(k)
    k2[5, :, 0] = _bf16(1.0)      # key of the second position: score 2 * scale, first: 0
    out = orc.decode_attention(q2, k2, v, [[4, 5]], [2], hq, hkv, scale)
    w1 = 1.0 / (1.0 + np.exp(-2.0 * scale))
    for h in range(hq):
        g = h // group
        assert np.allclose(out[0, h], w1 * vv[5, g] + (1 - w1) * vv[4, g], rtol=0, atol=1e-13)
    # one dominant score (exp(1000) overflows unless the maximum is subtracted first)
    q3 = np.zeros_like(q)
    q3[:, :, 0] = _bf16(1000.0)
    out = orc.decode_attention(q3, k2, v, [[1, 2, 5, 8]], [0], hq, hkv, 1.0)
    for h in range(hq):
        assert np.allclose(out[0, h], vv[5, h // group], rtol=0, atol=1e-13)
    # grouped heads: value rows constant per kv head give that head's constant
    vc = np.zeros_like(v)
    for g in range(hkv):
        vc[:, g, :] = _bf16(float(g + 1))
    out = orc.decode_attention(q, k, vc, [sl], [2], hq, hkv, scale)
    for h in range(hq):
        assert np.allclose(out[0, h], h // group + 1, rtol=0, atol=1e-13)
    # doubling every value doubles the output (2 v is exact in bf16)
    v2 = _bf16(2.0 * vv)
    a = orc.decode_attention(q, k, v, [sl], [1], hq, hkv, scale)
    b = orc.decode_attention(q, k, v2, [sl], [1], hq, hkv, scale)
    assert np.allclose(b, 2 * a, rtol=0, atol=1e-12)
    # physical placement does not matter: the same logical rows at other slots
    perm = rng.permutation(rows)
    kp, vp = np.empty_like(k), np.empty_like(v)
    kp[perm], vp[perm] = k, v            # row j moves to slot perm[j]
    a = orc.decode_attention(q, k, v, [sl, sl[::-1]], [0, 1], hq, hkv, scale)
    b = orc.decode_attention(q, kp, vp, [list(perm[sl]), list(perm[sl[::-1]])], [0, 1], hq,
                             hkv, scale)
    assert np.array_equal(a, b)
    # a slot of -1 holds no token
    c = orc.decode_attention(q, k, v, [[3, -1, 9, 11, -1, 20, 21, 33]], [0], hq, hkv, scale)
    e = orc.decode_attention(q, k, v, [sl], [0], hq, hkv, scale)
    assert np.array_equal(c, e)
    pin_attention_lse(orc, q, k, v, q2, k2, q3, sl, hq, hkv, scale)


def pin_attention_lse(orc, q, k, v, q2, k2, q3, sl, hq, hkv, scale):
    """The log of the softmax normalizer: closed forms, and the identity that merges attention
    over disjoint position sets (what context-parallel ranks combine)."""
    group = hq // hkv
    qv, kv_ = _bf16_value(q), _bf16_value(k)
    # one token: its score
    _, lse = orc.decode_attention(q, k, v, [[7]], [1], hq, hkv, scale, with_lse=True)
    for h in range(hq):
        assert np.isclose(lse[0, h], scale * float(np.dot(qv[1, h], kv_[7, h // group])),
                          rtol=0, atol=1e-13)
    # no token: -inf
    _, lse = orc.decode_attention(q, k, v, [[]], [1], hq, hkv, scale, with_lse=True)
    assert np.all(lse == -np.inf)
    # zero query: every score 0, so log n
    _, lse = orc.decode_attention(np.zeros_like(q), k, v, [sl], [0], hq, hkv, scale, with_lse=True)
    assert np.allclose(lse, np.log(len(sl)), rtol=0, atol=1e-14)
    # two one-hot keys: log(1 + e^(2 scale))
    _, lse = orc.decode_attention(q2, k2, v, [[4, 5]], [2], hq, hkv, scale, with_lse=True)
    assert np.allclose(lse, np.log1p(np.exp(2.0 * scale)), rtol=0, atol=1e-14)
    # a dominant score of 1000 among zeros: 1000 (exp(1000) overflows unless the max is taken out)
    _, lse = orc.decode_attention(q3, k2, v, [[1, 2, 5, 8]], [0], hq, hkv, 1.0, with_lse=True)
    assert np.allclose(lse, 1000.0, rtol=0, atol=1e-12)
    # merging attention over a split of the positions gives the whole: with L = logaddexp of the
    # parts' lse, out = sum exp(lse_part - L) out_part; an empty part (lse -inf) adds nothing
    full, lf = orc.decode_attention(q, k, v, [sl], [0], hq, hkv, scale, with_lse=True)
    for part_a in ([3, 11, 21], [3, 9, 11, 20, 21, 33], [33]):
        part_b = [s_ for s_ in sl if s_ not in part_a]
        oa, la = orc.decode_attention(q, k, v, [part_a], [0], hq, hkv, scale, with_lse=True)
        ob, lb = orc.decode_attention(q, k, v, [part_b], [0], hq, hkv, scale, with_lse=True)
        big = np.logaddexp(la, lb)
        with np.errstate(invalid="ignore"):
            wa = np.where(la == -np.inf, 0.0, np.exp(la - big))
            wb = np.where(lb == -np.inf, 0.0, np.exp(lb - big))
        merged = wa[..., None] * oa + wb[..., None] * ob
        assert np.allclose(merged, full, rtol=0, atol=1e-12)
        assert np.allclose(big, lf, rtol=0, atol=1e-12)


def pin_coordinates(orc):
    """Coordinate form == numpy row-major indexing of [layers][blocks][tokens] rows."""
    cfg = {f[0]: int(f[1]) for f in _lines("coordinate_layout.txt")}
    L, B, T, bpt = cfg["layers"], cfg["blocks"], cfg["tokens_per_block"], cfg["bytes_per_token"]
    rng = np.random.default_rng(3)
    pts = [(0, 0, 0), (L - 1, B - 1, T - 1), (1, 0, 0), (0, 1, 0), (0, 0, 1)]
    pts += [tuple(int(v) for v in (rng.integers(L), rng.integers(B), rng.integers(T)))
            for _ in range(200)]
    for (l, b, t) in pts:
        want = int(np.ravel_multi_index((l, b, t), (L, B, T))) * bpt
        assert orc.coord_offset(l, b, t, B, T, bpt) == want, (l, b, t)
    # the last row of that layout ends at 128 GiB: offsets need 64-bit integers
    assert orc.coord_offset(L - 1, B - 1, T - 1, B, T, bpt) + bpt == 128 << 30
    # element addresses of a real nested array
    shape = (3, 5, 4, 24)
    arr = np.zeros(shape, np.uint8)
    base = arr.ctypes.data
    for l in range(shape[0]):
        for b in range(shape[1]):
            for t in range(shape[2]):
                addr = arr[l, b, t].ctypes.data - base
                assert orc.coord_offset(l, b, t, shape[1], shape[2], shape[3]) == addr


def expected_caches_numpy(slots: np.ndarray, key: np.ndarray, value: np.ndarray,
                          num_blocks: int, block_size: int, sentinel: int):
    """Independent K/V scatter with numpy fancy indexing over [layers, B*T, row]."""
    L, M, E = key.shape
    kc = np.full((L, num_blocks * block_size, E), sentinel, key.dtype)
    vc = np.full_like(kc, sentinel)
    ok = (slots >= 0) & (slots < num_blocks * block_size)
    kc[:, slots[ok]] = key[:, ok]
    vc[:, slots[ok]] = value[:, ok]
    return kc, vc


def pin_kv_write(orc, workloads):
    """K/V scatter == numpy scatter; windows compose; pads and stray slots write nothing."""
    from workloads import BF16_SENTINEL
    for w in workloads:
        slots, _ = orc.slot_mapping_paged(w.query_start_loc, w.num_reqs, w.positions,
                                          w.max_num_tokens, w.block_table, w.num_blocks_per_req,
                                          w.block_size)
        key, value = w.kv_plane(0), w.kv_plane(1)
        ek, ev = expected_caches_numpy(slots, key, value, w.num_blocks, w.block_size,
                                       BF16_SENTINEL)
        rows = w.num_layers * w.num_blocks * w.block_size
        kc = np.full((rows, w.row_elems), BF16_SENTINEL, np.uint16)
        vc = np.full_like(kc, BF16_SENTINEL)
        f = orc.kv_write(slots, key, value, w.num_blocks, w.block_size, kc, vc)
        assert f == 0
        assert np.array_equal(kc, ek.reshape(rows, -1)), w.name
        assert np.array_equal(vc, ev.reshape(rows, -1)), w.name
        # piecewise windows give the same bytes
        kc2 = np.full_like(kc, BF16_SENTINEL)
        vc2 = np.full_like(kc, BF16_SENTINEL)
        cuts = np.unique(np.concatenate([[0, rows], np.random.default_rng(5).integers(
            0, rows, size=7)]))
        for a, b in zip(cuts[:-1], cuts[1:]):
            orc.kv_write(slots, key, value, w.num_blocks, w.block_size, kc2[a:b], vc2[a:b],
                         row_begin=int(a))
        assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)
        # K/V rows of padded tokens (bf16 1.0 everywhere) never reach the cache
        n = w.num_tokens
        if n < w.max_num_tokens:
            marker = key[0, n]
            assert not (kc == marker).all(axis=1).any()
    # a slot beyond the cache is skipped and flagged; a pad slot is skipped silently
    key = np.arange(2 * 3 * 8, dtype=np.uint16).reshape(2, 3, 8)
    kc = np.zeros((2 * 2 * 2, 8), np.uint16)
    vc = np.zeros_like(kc)
    f = orc.kv_write(np.array([3, 4, PAD]), key, key, 2, 2, kc, vc)
    assert f == 8
    assert (kc[3] == key[0, 0]).all() and (kc[4 + 3] == key[1, 0]).all()
    assert (np.delete(kc, [3, 7], axis=0) == 0).all()


def all_pins(orc, small, full=()):
    """Every pin, for the mutation campaign (small inputs only)."""
    pin_golden_bs16(orc)
    pin_figure6(orc)
    pin_fill_simulation(orc)
    pin_enumeration(orc)
    pin_padding_rules(orc)
    pin_range_equals_gather(orc, list(small) + list(full))
    pin_expansion(orc)
    pin_table_fill(orc, small)
    pin_context_parallel(orc, small)
    pin_coordinates(orc)
    pin_attention(orc)
    pin_kv_write(orc, small)
