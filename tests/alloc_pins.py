"""Checks that tie the allocator model (oracle/range_alloc.py) to facts outside itself.

  * hand-worked operation sequences (tests/golden/range_alloc_sequences.txt);
  * after every operation of seeded random sequences, recomputed from
    scratch: every usable block is free or held by exactly one live extent,
    extents are aligned and disjoint, the free runs are maximal, exported
    ranges equal the row's blocks compressed into runs of consecutive ids
    (tests/oracle_pins.py's _runs_of), a new extent lies at the lowest aligned
    start with enough free blocks (a brute-force scan of the free blocks
    before the call), evictions take the oldest cache-only extents and only
    as many as needed, and a failed call changes nothing;
  * growth in place keeps a lone growing request at one range.

The same driver (run_ops) runs the native allocator in the parity tests.
"""
from __future__ import annotations

import os
from typing import Callable, List, Tuple

import numpy as np

from oracle.range_alloc import INVALID, NO_SPACE, NOT_FOUND, OK, UNSUPPORTED
from oracle_pins import _runs_of

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "range_alloc_sequences.txt")
STATUS = {"OK": OK, "INVALID": INVALID, "UNSUPPORTED": UNSUPPORTED, "NO_SPACE": NO_SPACE,
          "NOT_FOUND": NOT_FOUND}


def apply(obj, op: Tuple) -> Tuple[int, int]:
    """Run one operation; returns (status, evicted count for 'evict' else 0)."""
    kind = op[0]
    if kind == "extend":
        return obj.extend(op[1], op[2]), 0
    if kind == "release":
        return obj.release(op[1]), 0
    if kind == "insert":
        return obj.cache_insert(op[1], op[2], op[3], op[4]), 0
    if kind == "acquire":
        return obj.cache_acquire(op[1], op[2]), 0
    if kind == "evict":
        return obj.cache_evict(op[1])
    raise ValueError(kind)


def golden_sequences():
    seqs, cur = [], None
    with open(GOLDEN) as f:
        for raw in f:
            line = raw.rstrip("\n")
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            words = line.split()
            if words[0] == "pool":
                cur = {"pool": tuple(int(x) for x in words[1:]), "steps": []}
                seqs.append(cur)
            elif line.startswith(" "):
                cur["steps"][-1][2].append(words)
            else:
                kind = words[0]
                nargs = {"extend": 2, "release": 1, "insert": 4, "acquire": 2, "evict": 1}[kind]
                args = [int(x) for x in words[1:1 + nargs]]
                status = STATUS[words[1 + nargs]]
                evicted = int(words[2 + nargs]) if len(words) > 2 + nargs else None
                cur["steps"].append(((kind, *args), (status, evicted), []))
    return seqs


def pin_golden(make: Callable):
    """Every hand-worked sequence, state by state; `make(num_blocks, A, first, rows)`."""
    for seq in golden_sequences():
        obj = make(*seq["pool"])
        for op, (status, evicted), checks in seq["steps"]:
            got, k = apply(obj, op)
            assert got == status, (seq["pool"], op, got, status)
            if evicted is not None:
                assert k == evicted, (op, k, evicted)
            for c in checks:
                if c[0] == "row":
                    want = [tuple(int(v) for v in x.split(":")) for x in c[2:]]
                    assert obj.row_extents(int(c[1])) == want, (op, c, obj.row_extents(int(c[1])))
                elif c[0] == "ranges":
                    want = [tuple(int(v) for v in x.split(":")) for x in c[2:]]
                    assert obj.row_ranges(int(c[1])) == want, (op, c, obj.row_ranges(int(c[1])))
                elif c[0] == "free":
                    want = [tuple(int(v) for v in x.split(":")) for x in c[1:]]
                    assert obj.free_runs() == want, (op, c, obj.free_runs())
                elif c[0] == "lru":
                    assert obj.lru_starts() == [int(x) for x in c[1:]], (op, c, obj.lru_starts())


def random_op(rng, obj, rows: int, A: int, max_chunks: int):
    """One operation drawn to exercise every path, some of them invalid on purpose."""
    u = rng.random()
    row = int(rng.integers(0, rows))
    if u < 0.45:
        n = A * int(rng.integers(0, max_chunks + 1))
        if rng.random() < 0.03:
            n += 1 if A > 1 else -1 - n   # not a multiple of A, or negative
        return ("extend", row, n)
    if u < 0.62:
        return ("release", row)
    if u < 0.80:
        size = sum(ln for _, ln in obj.row_extents(row))
        first = A * int(rng.integers(0, max(1, size // A + 1)))
        count = A * int(rng.integers(1, 4))
        if rng.random() < 0.05:
            first += 1
        return ("insert", int(rng.integers(0, 12)), row, first, count)
    if u < 0.95:
        return ("acquire", int(rng.integers(0, 14)), row)
    return ("evict", int(rng.integers(0, 3)))


def check_state(obj, A: int, num_blocks: int, usable: List[bool]):
    """Recompute what must hold after any operation, from the object's views only."""
    held = [0] * num_blocks
    seen = {}
    rows = obj.max_rows
    for r in range(rows):
        blocks = []
        for s, ln in obj.row_extents(r):
            assert s % A == 0 and ln % A == 0 and ln > 0
            seen[(s, ln)] = True
            blocks += list(range(s, s + ln))
        assert [tuple(x) for x in obj.row_ranges(r)] == _runs_of(blocks), r
    lru = obj.lru_starts()
    free = set()
    runs = obj.free_runs()
    for i, (s, ln) in enumerate(runs):
        assert ln > 0
        if i:
            assert runs[i - 1][0] + runs[i - 1][1] < s   # maximal: never adjacent
        free.update(range(s, s + ln))
    for (s, ln) in seen:
        for b in range(s, s + ln):
            held[b] += 1
    for b in range(num_blocks):
        assert not (b in free and held[b]), b
        assert held[b] <= 1, b
        if not usable[b]:
            assert b not in free and not held[b]
    st = obj.stats()
    assert st["free_blocks"] == len(free)
    cache_only = st["cache_only_blocks"]
    in_rows = sum(held)
    # usable blocks are free, listed by a row, or cache-only
    assert len(free) + in_rows + cache_only == sum(usable), (len(free), in_rows, cache_only)
    assert len(lru) == len(set(lru))


def run_ops(obj, ops) -> List[Tuple[int, int]]:
    return [apply(obj, op) for op in ops]


def snapshot(obj):
    return ([obj.row_extents(r) for r in range(obj.max_rows)], obj.free_runs(), obj.lru_starts(),
            obj.stats())


def pin_random(make: Callable, seeds=range(8), n_ops=400):
    """Random sequences on small pools, every rule re-derived after every operation."""
    for seed in seeds:
        rng = np.random.default_rng(9000 + seed)
        A = int(rng.choice([1, 1, 2, 4]))
        first = int(rng.integers(0, 3))
        num_blocks = int(rng.integers(24, 96))
        rows = int(rng.integers(2, 6))
        obj = make(num_blocks, A, first, rows)
        usable = [b < (num_blocks // A) * A and b >= -(-first // A) * A for b in range(num_blocks)]
        for i in range(n_ops):
            op = random_op(rng, obj, rows, A, max_chunks=6)
            before = snapshot(obj)
            free_before = {b for s, ln in obj.free_runs() for b in range(s, s + ln)}
            lru_before = obj.lru_extents()
            status, k = apply(obj, op)
            after = snapshot(obj)
            if status != OK:
                assert after == before, (seed, i, op, status)
            elif op[0] == "extend" and op[2] > 0:
                n = op[2]
                row_before = before[0][op[1]]
                row_after = after[0][op[1]]
                new = row_after[len(row_before):]
                evicted = [e for e in lru_before if e not in obj.lru_extents()]
                # evictions: the oldest ones, only when too few blocks were free, and no more
                # than needed (without the last one there would not have been enough)
                assert evicted == lru_before[:len(evicted)], (seed, i)
                if len(free_before) >= n:
                    assert not evicted, (seed, i)
                else:
                    assert len(free_before) + sum(ln for _, ln in evicted) >= n, (seed, i)
                    assert len(free_before) + sum(ln for _, ln in evicted[:-1]) < n, (seed, i)
                freed = set(free_before)
                if not evicted and len(new) > 1:
                    # no single run held n: the lowest runs, whole, in address order
                    runs_before = before[1]
                    assert all(ln < n for _, ln in runs_before), (seed, i)
                    assert new[:-1] == runs_before[:len(new) - 1], (seed, i)
                    last = runs_before[len(new) - 1]
                    assert new[-1] == (last[0], n - sum(ln for _, ln in new[:-1])), (seed, i)
                if not evicted and not new:
                    # grown in place: the last extent got longer by n
                    assert row_after[-1][1] == row_before[-1][1] + n, (seed, i)
                elif not evicted and len(new) == 1 and new[0][1] == n:
                    # first fit: no lower aligned start had n free blocks
                    s = new[0][0]
                    for t in range(0, s, A):
                        assert not all(b in freed for b in range(t, t + n)), (seed, i, t, s)
            check_state(obj, A, num_blocks, usable)


def pin_lone_growth(make: Callable):
    """A request growing alone (decode) keeps one range: growth happens in place."""
    for A in (1, 2, 4):
        obj = make(256, A, 1, 2)
        for step in range(40):
            assert obj.extend(0, A) == OK
            assert len(obj.row_ranges(0)) == 1 and len(obj.row_extents(0)) == 1
        assert obj.row_extents(0)[0][0] == -(-1 // A) * A
        assert obj.release(0) == OK
        assert obj.stats()["free_blocks"] == obj.stats()["usable_blocks"]
        assert len(obj.free_runs()) == 1


def pin_allocator(make: Callable, seeds=range(8)):
    pin_golden(make)
    pin_lone_growth(make)
    pin_random(make, seeds)
