"""Seeded generator of KV-cache write workloads.

Every workload is drawn from numpy ``Generator(PCG64)`` streams keyed by the
workload seed, so the same seed always yields the same bytes.  The recipe
follows the pages' workload descriptions:

* requests carry a context length after this step (``end``) and a number of
  tokens scheduled this step (``n_new``); their positions are the last
  ``n_new`` positions before ``end`` (a prefill chunk, or one decode token);
* each request owns ``ceil(end / block_size)`` physical blocks, grouped into
  contiguous runs ("ranges"); the block-table row is the concatenation of the
  runs in logical order, the range descriptors are the runs themselves
  (start, length, and the count of logical blocks before the run);
* block 0 is the reserved null block and is never handed out;
* when the pool cannot hold every request's blocks, the blocks that receive
  this step's tokens stay unique and unaliased and only older (history-only)
  blocks share physical ids with each other;
* K and V rows of real tokens are N(0, 1) rounded to bf16; rows of padded
  tokens hold bf16 1.0 so that a write of a padded token is detectable.

No slot id, cache offset or expected cache content is computed here.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

BF16_SENTINEL = 0x7FC0   # cache pre-fill; a bf16 NaN pattern, only ever compared as bytes
BF16_MARKER_ONE = 0x3F80  # bf16 1.0: payload of padded-token K/V rows

# RunSpec: ("len", lo, hi)  -> run lengths ~U[lo, hi], the last one truncated
#          ("count", lo, hi) -> number of runs ~U[lo, hi] (clamped), random cut points
#          ("equal", k)      -> k runs of equal length (k must divide the block count)
RunSpec = Tuple


@dataclass
class Request:
    end: int                      # context length after this step, in tokens
    n_new: int                    # scheduled tokens: positions [end - n_new, end)
    alloc_blocks: Optional[int] = None  # blocks owned; default ceil(end / block_size)


@dataclass
class Workload:
    name: str
    seed: int
    block_size: int               # unit of block_table and range descriptors
    kernel_block_size: int        # block size of the cache that kernels write
    num_blocks: int               # pool size per layer, in block_size units
    num_layers: int
    num_kv_heads: int
    head_dim: int
    max_num_tokens: int
    num_reqs: int                 # entries of query_start_loc minus one (incl. dummies)
    query_start_loc: np.ndarray   # int32 [num_reqs + 1]
    positions: np.ndarray         # int64 [max_num_tokens]; tail is garbage
    block_table: np.ndarray       # int32 [max_num_reqs, table_stride]
    num_blocks_per_req: np.ndarray  # int32 [max_num_reqs]
    range_start: np.ndarray       # int32 [max_num_reqs, range_stride]
    range_len: np.ndarray         # int32 [max_num_reqs, range_stride]
    range_cum: np.ndarray         # int32 [max_num_reqs, range_stride]
    num_ranges: np.ndarray        # int32 [max_num_reqs]
    requests: List[Request] = field(default_factory=list)
    description: str = ""

    # ---- derived sizes -------------------------------------------------
    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[self.num_reqs])

    @property
    def max_num_reqs(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def table_stride(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def range_stride(self) -> int:
        return int(self.range_start.shape[1])

    @property
    def bytes_per_token(self) -> int:
        return self.num_kv_heads * self.head_dim * 2

    @property
    def row_elems(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def blocks_per_kv_block(self) -> int:
        return self.block_size // self.kernel_block_size

    @property
    def kernel_num_blocks(self) -> int:
        return self.num_blocks * self.blocks_per_kv_block

    @property
    def cache_rows_per_layer(self) -> int:
        return self.num_blocks * self.block_size

    def describe(self) -> str:
        return (f"{self.name}: seed={self.seed} reqs={self.num_reqs} tokens={self.num_tokens}/"
                f"{self.max_num_tokens} bs={self.block_size}->{self.kernel_block_size} "
                f"pool={self.num_blocks} layers={self.num_layers} row={self.bytes_per_token}B "
                f"table={self.max_num_reqs}x{self.table_stride} ranges<= {self.range_stride}")

    # ---- K/V payload ---------------------------------------------------
    def kv_layer(self, plane: int, layer: int) -> np.ndarray:
        """bf16 bit patterns [max_num_tokens, H*D] of K (plane 0) or V (plane 1)."""
        rng = np.random.Generator(np.random.PCG64([self.seed, 17 + plane, layer]))
        n_real = self.num_tokens
        out = np.empty((self.max_num_tokens, self.row_elems), dtype=np.uint16)
        if n_real:
            out[:n_real] = _bf16_normal(rng, n_real * self.row_elems).reshape(n_real, self.row_elems)
        out[n_real:] = BF16_MARKER_ONE
        return out

    def kv_plane(self, plane: int) -> np.ndarray:
        """bf16 bit patterns [num_layers, max_num_tokens, H*D]."""
        out = np.empty((self.num_layers, self.max_num_tokens, self.row_elems), dtype=np.uint16)
        for layer in range(self.num_layers):
            out[layer] = self.kv_layer(plane, layer)
        return out


def _bf16_normal(rng: np.random.Generator, n: int) -> np.ndarray:
    """n draws of N(0,1) in float32, rounded to bf16 (nearest, ties to even)."""
    x = rng.standard_normal(n, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _split_runs(rng: np.random.Generator, nb: int, spec: RunSpec) -> List[int]:
    if nb <= 0:
        return []
    kind = spec[0]
    if kind == "len":
        lo, hi = spec[1], spec[2]
        runs, left = [], nb
        while left > 0:
            ln = min(int(rng.integers(lo, hi + 1)), left)
            runs.append(ln)
            left -= ln
        return runs
    if kind == "count":
        k = int(rng.integers(spec[1], spec[2] + 1))
        k = max(1, min(k, nb))
        if k == 1:
            return [nb]
        cuts = np.sort(rng.choice(np.arange(1, nb), size=k - 1, replace=False))
        edges = np.concatenate([[0], cuts, [nb]])
        return [int(v) for v in np.diff(edges)]
    if kind == "equal":
        k = spec[1]
        if nb % k:
            raise ValueError(f"equal runs: {k} does not divide {nb} blocks")
        return [nb // k] * k
    raise ValueError(f"unknown run spec {spec!r}")


def _composition(rng: np.random.Generator, total: int, parts: int) -> np.ndarray:
    """Random split of `total` into `parts` non-negative integers."""
    if parts <= 0:
        return np.zeros(0, dtype=np.int64)
    if total == 0 or parts == 1:
        out = np.zeros(parts, dtype=np.int64)
        out[-1] = total
        return out
    cuts = np.sort(rng.integers(0, total + 1, size=parts - 1))
    return np.diff(np.concatenate([[0], cuts, [total]]))


def _place(rng: np.random.Generator, runs: List[List[int]], writes: List[List[bool]],
           num_blocks: int) -> List[List[List[Tuple[int, int]]]]:
    """Assign each run a physical placement: a list of (start, length) pieces.

    Ids are drawn from [1, num_blocks); block 0 stays the null block.
    """
    usable = num_blocks - 1
    flat = [(r, j, ln) for r, rr in enumerate(runs) for j, ln in enumerate(rr)]
    total = sum(x[2] for x in flat)
    pieces: List[List[List[Tuple[int, int]]]] = [[[] for _ in rr] for rr in runs]
    if total <= usable:
        order = rng.permutation(len(flat))
        gaps = _composition(rng, usable - total, len(flat) + 1)
        cur = 1
        for gi, idx in enumerate(order):
            cur += int(gaps[gi])
            r, j, ln = flat[idx]
            pieces[r][j] = [(cur, ln)]
            cur += ln
        return pieces
    # Over-subscribed pool: runs that receive this step's tokens are placed
    # first, disjointly; history-only runs then fill the remaining spans
    # cyclically and may share ids with each other (never with a written run).
    wr = [x for x in flat if writes[x[0]][x[1]]]
    hist = [x for x in flat if not writes[x[0]][x[1]]]
    w_total = sum(x[2] for x in wr)
    if w_total > usable:
        raise ValueError("pool too small for the blocks written this step")
    order = rng.permutation(len(wr))
    gaps = _composition(rng, usable - w_total, len(wr) + 1)
    spans: List[Tuple[int, int]] = []
    cur = 1
    for gi, idx in enumerate(order):
        g = int(gaps[gi])
        if g:
            spans.append((cur, cur + g))
        cur += g
        r, j, ln = wr[idx]
        pieces[r][j] = [(cur, ln)]
        cur += ln
    if int(gaps[-1]):
        spans.append((cur, cur + int(gaps[-1])))
    if hist and not spans:
        raise ValueError("no free span left for history blocks")
    si, pos = 0, spans[0][0] if spans else 0
    for idx in rng.permutation(len(hist)):
        r, j, ln = hist[idx]
        left = ln
        while left > 0:
            a, b = spans[si]
            take = min(left, b - pos)
            pieces[r][j].append((pos, take))
            pos += take
            left -= take
            if pos == b:
                si = (si + 1) % len(spans)
                pos = spans[si][0]
    return pieces


def custom(name: str, seed: int, requests: Sequence[Request], *, block_size: int,
           num_blocks: int, runs: RunSpec, num_layers: int = 1, num_kv_heads: int = 8,
           head_dim: int = 128, max_num_tokens: Optional[int] = None,
           table_stride: Optional[int] = None, range_stride: Optional[int] = None,
           dummy_reqs: int = 0, kernel_block_size: Optional[int] = None,
           description: str = "") -> Workload:
    """Build a workload from explicit requests (in batch order)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    bs = block_size
    nbs, run_lists, write_lists = [], [], []
    for rq in requests:
        if rq.n_new < 0 or rq.n_new > rq.end:
            raise ValueError(f"bad request {rq}")
        nb = rq.alloc_blocks if rq.alloc_blocks is not None else -(-rq.end // bs)
        rl = _split_runs(rng, nb, runs)
        # logical block interval that holds this step's tokens (allocation bookkeeping)
        lo_b = (rq.end - rq.n_new) // bs
        hi_b = (rq.end - 1) // bs if rq.n_new else -1
        cum, wl = 0, []
        for ln in rl:
            wl.append(rq.n_new > 0 and cum <= hi_b and lo_b < cum + ln)
            cum += ln
        nbs.append(nb)
        run_lists.append(rl)
        write_lists.append(wl)
    placed = _place(rng, run_lists, write_lists, num_blocks)

    n_real = len(requests)
    max_reqs = n_real + dummy_reqs
    t_stride = table_stride if table_stride is not None else max(1, max(nbs, default=1))
    piece_counts = [sum(len(p) for p in pr) for pr in placed]
    r_stride = range_stride if range_stride is not None else max(1, max(piece_counts, default=1))
    if max(nbs, default=0) > t_stride:
        raise ValueError("table stride too small")
    if max(piece_counts, default=0) > r_stride:
        raise ValueError(f"range stride {r_stride} too small for {max(piece_counts)} runs")

    table = np.zeros((max_reqs, t_stride), dtype=np.int32)
    nbpr = np.zeros(max_reqs, dtype=np.int32)
    rs = np.zeros((max_reqs, r_stride), dtype=np.int32)
    rlen = np.zeros((max_reqs, r_stride), dtype=np.int32)
    rcum = np.zeros((max_reqs, r_stride), dtype=np.int32)
    nr = np.zeros(max_reqs, dtype=np.int32)
    for r in range(n_real):
        ids: List[int] = []
        k = 0
        for run_pieces in placed[r]:
            for (st, ln) in run_pieces:
                rs[r, k], rlen[r, k], rcum[r, k] = st, ln, len(ids)
                ids.extend(range(st, st + ln))
                k += 1
        nr[r] = k
        nbpr[r] = len(ids)
        table[r, :len(ids)] = ids

    counts = [rq.n_new for rq in requests] + [0] * dummy_reqs
    qsl = np.zeros(max_reqs + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(counts)
    n_tok = int(qsl[-1])
    m = max_num_tokens if max_num_tokens is not None else n_tok
    if m < n_tok:
        raise ValueError("max_num_tokens below the scheduled token count")
    pos = np.empty(m, dtype=np.int64)
    t = 0
    for rq in requests:
        pos[t:t + rq.n_new] = np.arange(rq.end - rq.n_new, rq.end, dtype=np.int64)
        t += rq.n_new
    # positions past num_tokens are ignored: fill with garbage
    pos[n_tok:] = rng.integers(-(1 << 40), 1 << 40, size=m - n_tok, dtype=np.int64)

    return Workload(name=name, seed=seed, block_size=bs,
                    kernel_block_size=kernel_block_size or bs, num_blocks=num_blocks,
                    num_layers=num_layers, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    max_num_tokens=m, num_reqs=max_reqs, query_start_loc=qsl, positions=pos,
                    block_table=table, num_blocks_per_req=nbpr, range_start=rs, range_len=rlen,
                    range_cum=rcum, num_ranges=nr, requests=list(requests),
                    description=description)


# ---------------------------------------------------------------------------
# The five workloads of the write-path study.
# ---------------------------------------------------------------------------
CONFIG_NAMES = ("tiny_prefill", "decode_step", "mixed_chunked", "long_context", "full_32_layer")


def tiny_prefill(seed: int = 4601) -> Workload:
    """4 prompts {7,33,100,250} (390 tokens) padded to 512; bs 16; pool 512; 1-3 runs each."""
    reqs = [Request(n, n) for n in (7, 33, 100, 250)]
    return custom("tiny_prefill", seed, reqs, block_size=16, num_blocks=512, runs=("count", 1, 3),
                  max_num_tokens=512, table_stride=16, range_stride=4,
                  description="tiny prefill, 1 layer, 8x128 bf16")


def decode_step(seed: int = 4602, num_reqs: int = 256, max_ctx: int = 8192,
                num_blocks: int = 65536) -> Workload:
    """256 decodes, context ~U[1,8192] (incl. the new token); runs ~U[1,64]; pool 65,536."""
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    ctx = rng.integers(1, max_ctx + 1, size=num_reqs)
    reqs = [Request(int(c), 1) for c in ctx]
    stride = -(-max_ctx // 16)
    return custom("decode_step", seed, reqs, block_size=16, num_blocks=num_blocks,
                  runs=("len", 1, 64), table_stride=stride, range_stride=stride,
                  description="decode step, 1 layer, Llama-3-8B KV shape")


def mixed_chunked(seed: int = 4603, num_prefill: int = 8, num_decode: int = 56,
                  total_tokens: int = 8192, max_prior: int = 32768,
                  chunk_lo: int = 512, chunk_hi: int = 2048, num_blocks: int = 131072) -> Workload:
    """8 prefill chunks of 512-2048 tokens + 56 decodes = 8192 tokens; 1-128 runs each."""
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    chunk_total = total_tokens - num_decode
    while True:
        extra = _composition(rng, chunk_total - num_prefill * chunk_lo, num_prefill)
        chunks = chunk_lo + extra
        if chunks.max() <= chunk_hi:
            break
    reqs = []
    for c in chunks:
        prior = int(rng.integers(0, max_prior + 1))
        reqs.append(Request(prior + int(c), int(c)))
    for _ in range(num_decode):
        reqs.append(Request(int(rng.integers(1, max_prior + 1)), 1))
    reqs = [reqs[i] for i in rng.permutation(len(reqs))]
    stride = -(-(max_prior + chunk_hi) // 16)
    return custom("mixed_chunked", seed, reqs, block_size=16, num_blocks=num_blocks,
                  runs=("count", 1, 128), table_stride=stride, range_stride=128,
                  description="mixed chunked-prefill batch, 1 layer")


def long_context(ranges_per_req: int = 1, seed: int = 4604, num_reqs: int = 16,
                 context: int = 131072, chunk: int = 8192, manager_block_size: int = 32,
                 kernel_block_size: int = 16, range_stride: int = 4096) -> Workload:
    """16 requests at 128K context, 8192-token chunk each; manager bs 32 -> kernel bs 16.

    Every request owns context/32 manager blocks split into `ranges_per_req`
    equal runs; the pool holds exactly those blocks plus the null block.
    """
    nb = context // manager_block_size
    reqs = [Request(context, chunk) for _ in range(num_reqs)]
    return custom(f"long_context_r{ranges_per_req}", seed * 10000 + ranges_per_req, reqs,
                  block_size=manager_block_size, num_blocks=num_reqs * nb + 1,
                  runs=("equal", ranges_per_req), table_stride=nb,
                  range_stride=max(range_stride, ranges_per_req),
                  kernel_block_size=kernel_block_size,
                  description=f"128K context, {ranges_per_req} ranges per request")


def full_32_layer(seed: int = 4605, num_layers: int = 32, num_prefill: int = 128,
                  prefill_chunk: int = 125, num_decode: int = 384, max_ctx: int = 16384,
                  num_blocks: int = 32768, runs: RunSpec = ("len", 1, 64)) -> Workload:
    """512 requests (128 prefill chunks of 125 tokens + 384 decodes) = 16,384 tokens x 32 layers."""
    rng = np.random.Generator(np.random.PCG64([seed, 0]))
    reqs = [Request(int(rng.integers(prefill_chunk, max_ctx + 1)), prefill_chunk)
            for _ in range(num_prefill)]
    reqs += [Request(int(rng.integers(1, max_ctx + 1)), 1) for _ in range(num_decode)]
    reqs = [reqs[i] for i in rng.permutation(len(reqs))]
    stride = -(-max_ctx // 16)
    return custom("full_32_layer", seed, reqs, block_size=16, num_blocks=num_blocks,
                  runs=runs, num_layers=num_layers, table_stride=stride,
                  range_stride=stride, description="32-layer write in one launch")


def config(name: str, **kw) -> Workload:
    """One of the five study workloads by name (long_context takes ranges_per_req)."""
    fn = {"tiny_prefill": tiny_prefill, "decode_step": decode_step,
          "mixed_chunked": mixed_chunked, "long_context": long_context,
          "full_32_layer": full_32_layer}[name]
    return fn(**kw)


def small_cases() -> List[Workload]:
    """Small workloads (seconds for the oracle) spanning many tiles and ragged tails."""
    cases: List[Workload] = [tiny_prefill()]
    rng = np.random.Generator(np.random.PCG64([4700, 0]))

    def mixed(seed, n_pref, n_dec, bs, max_ctx, **kw):
        r = np.random.Generator(np.random.PCG64([seed, 0]))
        reqs = []
        for _ in range(n_pref):
            c = int(r.integers(1, 300))
            reqs.append(Request(int(r.integers(0, max_ctx)) + c, c))
        for _ in range(n_dec):
            reqs.append(Request(int(r.integers(1, max_ctx)), 1))
        reqs = [reqs[i] for i in r.permutation(len(reqs))]
        return reqs

    reqs = mixed(4701, 6, 40, 16, 3000)
    n = sum(q.n_new for q in reqs)
    cases.append(custom("small_mixed_l3", 4701, reqs, block_size=16, num_blocks=700,
                        runs=("len", 1, 9), num_layers=3, max_num_tokens=n + 37))
    for bs in (1, 8, 64):
        reqs = mixed(4702 + bs, 3, 20, bs, 700)
        need = sum(-(-q.end // bs) for q in reqs)
        cases.append(custom(f"small_bs{bs}", 4702 + bs, reqs, block_size=bs,
                            num_blocks=need + 50, runs=("count", 1, 6),
                            max_num_tokens=sum(q.n_new for q in reqs) + 5))
    # over-subscribed pool: only written blocks stay unique
    reqs = mixed(4710, 4, 60, 16, 4000)
    cases.append(custom("small_oversub", 4710, reqs, block_size=16, num_blocks=600,
                        runs=("len", 1, 16), num_layers=2,
                        max_num_tokens=sum(q.n_new for q in reqs) + 64))
    # dummy (padded) requests with no tokens and NULL rows
    reqs = mixed(4711, 3, 10, 16, 1000)
    cases.append(custom("small_dummy", 4711, reqs, block_size=16, num_blocks=1024,
                        runs=("count", 1, 4), dummy_reqs=7,
                        max_num_tokens=sum(q.n_new for q in reqs) + 100))
    # positions past the allocated blocks (out-of-range padding)
    reqs = [Request(200, 200, alloc_blocks=5), Request(90, 1, alloc_blocks=3),
            Request(64, 64, alloc_blocks=4), Request(33, 10, alloc_blocks=0)]
    cases.append(custom("small_out_of_range", 4712, reqs, block_size=16, num_blocks=256,
                        runs=("count", 1, 3), table_stride=16, max_num_tokens=300))
    # nothing scheduled: every slot is padding, nothing is written
    cases.append(custom("small_empty", 4713, [Request(50, 0), Request(7, 0)], block_size=16,
                        num_blocks=64, runs=("count", 1, 2), max_num_tokens=130))
    # row widths other than 2048 bytes
    for (h, d) in ((1, 8), (2, 64), (12, 128), (16, 128), (4, 24)):
        reqs = mixed(4720 + h * 7 + d, 3, 12, 16, 900)
        cases.append(custom(f"small_row{h * d * 2}", 4720 + h * 7 + d, reqs, block_size=16,
                            num_blocks=600, runs=("count", 1, 5), num_kv_heads=h,
                            head_dim=d, num_layers=2,
                            max_num_tokens=sum(q.n_new for q in reqs) + 3))
    # scaled-down versions of the study workloads
    cases.append(decode_step(seed=4730, num_reqs=48, max_ctx=2048, num_blocks=4096))
    cases[-1].name = "small_decode"
    cases.append(mixed_chunked(seed=4731, num_prefill=3, num_decode=21, total_tokens=1600,
                               max_prior=4096, chunk_lo=100, chunk_hi=900, num_blocks=4096))
    cases[-1].name = "small_chunked"
    for r in (1, 4, 64):
        w = long_context(ranges_per_req=r, seed=4732, num_reqs=3, context=2048, chunk=700,
                         range_stride=64)
        w.name = f"small_long_r{r}"
        cases.append(w)
    cases.append(full_32_layer(seed=4733, num_layers=4, num_prefill=6, prefill_chunk=25,
                               num_decode=40, max_ctx=3000, num_blocks=400,
                               runs=("len", 1, 6)))
    cases[-1].name = "small_layers"
    del rng
    return cases


def range_tables(seed: int, runs_per_row: Sequence[int], *, max_len: int = 3,
                 max_start: int = 1 << 20, range_stride: Optional[int] = None):
    """Bare range descriptors (start, len, cum, num_ranges) for the table fill.

    Row r holds runs_per_row[r] runs with lengths drawn from [1, max_len] and
    starts drawn from [0, max_start); cum is the running count of blocks
    before each run (the descriptor precondition).  Runs may overlap: a
    table fill does not need unique blocks.  Entries past a row's count are 0.
    """
    rng = np.random.Generator(np.random.PCG64([seed, 3]))
    rows = len(runs_per_row)
    stride = range_stride if range_stride is not None else max(1, max(runs_per_row, default=1))
    start = np.zeros((rows, stride), np.int32)
    length = np.zeros((rows, stride), np.int32)
    cum = np.zeros((rows, stride), np.int32)
    num = np.zeros(rows, np.int32)
    for r, n in enumerate(runs_per_row):
        if n > stride:
            raise ValueError("range_stride too small")
        ln = rng.integers(1, max_len + 1, size=n)
        start[r, :n] = rng.integers(0, max_start, size=n)
        length[r, :n] = ln
        cum[r, :n] = np.concatenate([[0], np.cumsum(ln)[:-1]]) if n else []
        num[r] = n
    return start, length, cum, num


def decode_inputs(w: Workload, num_q_heads: int, seed: int, rows=None, num_kv_heads=None,
                  head_dim=None, kind: str = "normal"):
    """Queries, context lengths and cache contents for decode attention over w's layout.

    q: bf16 bits [num_reqs][num_q_heads][head_dim]; context_lens: the context of every real
    request (its `end`), 0 for dummy requests.  K and V rows [rows][num_kv_heads][head_dim]
    are drawn for the given cache rows (all rows of the pool when None) and returned with the
    row ids; every other row is left to the caller (zeros).  kind "normal": K, V ~ N(0, 1);
    kind "integers": K = 0 and V uniform on the integers -8 .. 8 (all exact in bf16).
    """
    hkv = num_kv_heads or w.num_kv_heads
    d = head_dim or w.head_dim
    rng = np.random.Generator(np.random.PCG64([seed, 5]))
    q = _bf16_normal(rng, w.num_reqs * num_q_heads * d).reshape(w.num_reqs, num_q_heads, d)
    ctx = np.zeros(w.num_reqs, np.int32)
    for r, rq in enumerate(w.requests):
        ctx[r] = rq.end
    if rows is None:
        rows = np.arange(w.num_blocks * w.block_size, dtype=np.int64)
    rows = np.asarray(rows, np.int64)
    shape = (len(rows), hkv, d)
    if kind == "normal":
        k = _bf16_normal(rng, len(rows) * hkv * d).reshape(shape)
        v = _bf16_normal(rng, len(rows) * hkv * d).reshape(shape)
    elif kind == "integers":
        k = np.zeros(shape, np.uint16)
        ints = rng.integers(-8, 9, size=shape, dtype=np.int32).astype(np.float32)
        v = (ints.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    else:
        raise ValueError(f"unknown kind {kind!r}")
    return q, ctx, rows, k, v
