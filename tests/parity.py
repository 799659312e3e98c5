"""Helpers for comparing the HIP path with the CPU oracle on the same seeded inputs.

Inputs come from `workloads`; expected values come only from `oracle`.  The
GPU side is reached only through the C-ABI binding (paged_kv_cache_46_amd).
"""
from __future__ import annotations

import sys
from typing import Dict, Optional, Tuple

import numpy as np
import torch

import oracle
import paged_kv_cache_46_amd as kvw
from workloads import BF16_SENTINEL, Workload

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    out = t.detach().cpu().numpy()
    return out.view(np.uint16) if out.dtype == np.int16 else out


class DeviceInputs:
    """The workload's mapping inputs on the GPU."""

    def __init__(self, w: Workload):
        self.qsl = dev(w.query_start_loc)
        self.positions = dev(w.positions)
        self.block_table = dev(w.block_table)
        self.nbpr = dev(w.num_blocks_per_req)
        self.rs, self.rl, self.rc = dev(w.range_start), dev(w.range_len), dev(w.range_cum)
        self.nr = dev(w.num_ranges)


def new_flag() -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def oracle_slots(w: Workload, variant: str, **over) -> Tuple[np.ndarray, int]:
    orc = oracle.get()
    bs = over.get("block_size", w.block_size)
    if variant == "paged":
        return orc.slot_mapping_paged(over.get("qsl", w.query_start_loc), w.num_reqs,
                                      w.positions, w.max_num_tokens,
                                      over.get("block_table", w.block_table),
                                      over.get("nbpr", w.num_blocks_per_req), bs)
    return orc.slot_mapping_ranges(over.get("qsl", w.query_start_loc), w.num_reqs, w.positions,
                                   w.max_num_tokens, over.get("rs", w.range_start),
                                   over.get("rl", w.range_len), over.get("rc", w.range_cum),
                                   over.get("nr", w.num_ranges), bs)


def gpu_slots(w: Workload, d: DeviceInputs, variant: str) -> Tuple[np.ndarray, int]:
    out = torch.full((w.max_num_tokens,), 12345, dtype=torch.int64, device=DEV)
    flag = new_flag()
    if variant == "paged":
        kvw.kvw_slot_mapping_paged(d.qsl, w.num_reqs, d.positions, w.max_num_tokens,
                                   d.block_table, d.nbpr, w.block_size, out, flag)
    else:
        kvw.kvw_slot_mapping_ranges(d.qsl, w.num_reqs, d.positions, w.max_num_tokens, d.rs, d.rl,
                                    d.rc, d.nr, w.block_size, out, flag)
    torch.cuda.synchronize()
    return host(out), int(flag.item())


class Caches:
    """K and V cache planes [layers * num_blocks * block_size, row] pre-filled with the sentinel."""

    def __init__(self, layers: int, num_blocks: int, block_size: int, row_elems: int):
        self.rows = layers * num_blocks * block_size
        self.row_elems = row_elems
        self.t = torch.full((2, self.rows, row_elems), BF16_SENTINEL, dtype=torch.int16, device=DEV)
        self.k, self.v = self.t[0], self.t[1]


def kv_device(w: Workload):
    key = dev(w.kv_plane(0)).view(w.num_layers, w.max_num_tokens, w.num_kv_heads, w.head_dim)
    value = dev(w.kv_plane(1)).view(w.num_layers, w.max_num_tokens, w.num_kv_heads, w.head_dim)
    return key, value


_WINDOWS: Dict[int, tuple] = {}


def _windows(rows: int, row_elems: int):
    """Host buffers of at least `rows` rows for one comparison window, kept across calls (per
    row width, largest so far): first touches of fresh pages took most of the time of a
    whole-cache comparison (a 128K cache plane is 4 GiB)."""
    have = _WINDOWS.get(row_elems)
    if have is None or have[0].shape[0] < rows:
        _WINDOWS.pop(row_elems, None)
        ek = np.empty((rows, row_elems), np.uint16)
        ev = np.empty_like(ek)
        staged = torch.empty((rows, row_elems), dtype=torch.int16, pin_memory=True)
        _WINDOWS[row_elems] = (ek, ev, staged)
    return _WINDOWS[row_elems]


def _words(a: np.ndarray) -> np.ndarray:
    """A flat view in the widest unsigned words the row width allows (faster equality)."""
    flat = a.reshape(-1)
    return flat.view(np.uint64) if flat.nbytes % 8 == 0 else flat


def compare_caches(w: Workload, caches: Caches, slots_oracle: np.ndarray, key_h: np.ndarray,
                   value_h: np.ndarray, num_blocks: int, block_size: int,
                   window_rows: int = 1 << 19) -> int:
    """Bytewise comparison of both cache planes against oracle windows; returns oracle flags.

    Each window of rows is written by the oracle into sentinel-filled host buffers and
    compared with the same rows copied from the device."""
    orc = oracle.get()
    flags = 0
    rows = caches.rows
    win = max(1, min(window_rows, rows))
    ek_all, ev_all, staged = _windows(win, caches.row_elems)
    for a in range(0, rows, win):
        b = min(rows, a + win)
        ek, ev = ek_all[:b - a], ev_all[:b - a]
        ek.fill(BF16_SENTINEL)
        ev.fill(BF16_SENTINEL)
        flags |= orc.kv_write(slots_oracle, key_h, value_h, num_blocks, block_size, ek, ev,
                              row_begin=a)
        for plane, name, exp in ((caches.k, "K", ek), (caches.v, "V", ev)):
            st = staged[:b - a]
            st.copy_(plane[a:b])
            got = st.numpy().view(np.uint16)
            if not np.array_equal(_words(got), _words(exp)):
                bad = np.nonzero((got != exp).any(axis=1))[0]
                raise AssertionError(f"{w.name}: {name} cache differs at {len(bad)} rows, first "
                                     f"row {a + int(bad[0])}")
    return flags
