"""Decode attention over the paged cache: HIP path vs CPU oracle (needs an MI355X).

The read side of the method: each request's query attends its context positions
0 .. n-1, whose slots the kernel resolves again from the block table (paged) or
from the range descriptors (range arithmetic).  The expected slots come from the
oracle's own slot mapping over those positions; the expected output from the
oracle's fp64 attention over the same slots.  Expected flag words are the oracle
slot mapping's, plus KVW_FLAG_COUNT where a context length is clamped and
KVW_FLAG_SLOT_OOB where a slot lies past the cache (such positions are skipped).

Tolerance: the kernel works in fp32 (unit roundoff u = 2^-24) from exact bf16
inputs, in base-2 exponent units (scores s = log2(e) * scale * q.k).  Its
summation structure: chunks of P = 256, 512, 1024 or 2048 positions; in a chunk four lane
groups each fold P/4 positions into a running (max m, sum l, weighted values acc),
moving m only when it grows by more than 8, so a group rescales at most
R = 1 + ceil(2S/8) times, S = log2(e) * scale * |q| * max_j |k_j| bounding |s|;
the groups are merged in two steps and the C = ceil(n/P) chunks in a second
launch.  To first order in u the output error is then at most
    u * max|V| * (P/2 + 6R + 2C + 60 + 20S),
taken at P = 2048 for the first term and P = 256 for C, so that it holds for
every chunk length:
per (request, query head): P/4 + R + C + 5 roundings along the numerator's
longest chain and P/4 + R + C + 12 along the denominator's, 2u per base-2
exponential (each p, and the R + 3 rescale factors a term can meet), and the
score error (4 two-term dot steps, 4 row adds, the scale product and the
subtraction of m: at most u(12S + 8) in log2 units, each weight moving by ln 2
times that, twice).  With 4 or 8 query heads per key/value head the kernel takes
q.k on matrix cores, a 128-term fp32 accumulation whose order the hardware fixes,
so the score error is taken as u(129S + 8) and the last term becomes 190S.  The
bound is written out in `tolerance` below.  Requests with no readable position
must give exactly 0.

The bound grows with the context, so at 128K a single dropped position would hide
under it.  The "integers" inputs close that gap bit-exactly: with K = 0 every
weight is exactly 1, and with V on the small integers every fp32 sum the kernel
forms is an exact integer, so out * n (n the readable positions) must round to the
oracle's integer sum in every dimension; a position dropped, read twice or read
from the wrong slot changes that sum.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_46_amd as kvw
from parity import DEV, dev, host, new_flag, say
from workloads import Request, config, custom, decode_inputs, long_context

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
FLAG_COUNT, FLAG_BAD_BLOCK, FLAG_SLOT_OOB = 2, 4, 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvw.library()
    yield
    torch.cuda.synchronize()


def f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


class Layout:
    """What the slots are resolved from: a block table or range descriptors, at block_size."""

    def __init__(self, w, block_size=None, table=None, nbpr=None, rs=None, rl=None, rc=None,
                 nr=None, num_blocks=None):
        self.bs = block_size or w.block_size
        self.num_blocks = num_blocks if num_blocks is not None else w.num_blocks
        self.table = w.block_table if table is None else table
        self.nbpr = w.num_blocks_per_req if nbpr is None else nbpr
        self.rs = w.range_start if rs is None else rs
        self.rl = w.range_len if rl is None else rl
        self.rc = w.range_cum if rc is None else rc
        self.nr = w.num_ranges if nr is None else nr

    @property
    def rows(self) -> int:
        return self.num_blocks * self.bs


def expected_slots(lay: Layout, mode: str, ctx: np.ndarray):
    """Per request, the slots of positions 0 .. ctx[r]-1 by the oracle's slot mapping (slots past
    the cache become -1 and raise KVW_FLAG_SLOT_OOB), and the flag word."""
    orc = oracle.get()
    num_reqs = len(ctx)
    qsl = np.zeros(num_reqs + 1, np.int32)
    qsl[1:] = np.cumsum(ctx)
    m = int(qsl[-1])
    if m == 0:
        return [np.zeros(0, np.int64) for _ in range(num_reqs)], 0
    pos = np.concatenate([np.arange(c, dtype=np.int64) for c in ctx])
    if mode == "paged":
        slots, flags = orc.slot_mapping_paged(qsl, num_reqs, pos, m, lay.table, lay.nbpr, lay.bs)
    else:
        slots, flags = orc.slot_mapping_ranges(qsl, num_reqs, pos, m, lay.rs, lay.rl, lay.rc,
                                               lay.nr, lay.bs)
    slots = slots.copy()
    past = slots >= lay.rows
    if past.any():
        slots[past] = -1
        flags |= FLAG_SLOT_OOB
    return [slots[qsl[r]:qsl[r + 1]] for r in range(num_reqs)], flags


def run_gpu(mode, lay: Layout, q, ctx_given, max_context, kc, vc, scale=None, num_reqs=None,
            chunk=0):
    num_reqs = q.shape[0] if num_reqs is None else num_reqs
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
    flag = new_flag()
    common = dict(q=dev(q), k_cache=kc, v_cache=vc, context_lens=dev(np.asarray(ctx_given,
                                                                              np.int32)),
                  max_context=max_context, num_blocks=lay.num_blocks, block_size=lay.bs, out=out,
                  scale=scale, err_flag=flag, chunk_positions=chunk)
    if mode == "paged":
        kvw.kvw_decode_attention(mode=kvw.KVW_SLOTS_PAGED, block_table=dev(lay.table),
                                 num_blocks_per_req=dev(lay.nbpr), **common)
    else:
        kvw.kvw_decode_attention(mode=kvw.KVW_SLOTS_RANGES, range_start=dev(lay.rs),
                                 range_len=dev(lay.rl), range_cum=dev(lay.rc),
                                 num_ranges=dev(lay.nr), **common)
    torch.cuda.synchronize()
    return host(out), int(flag.item())


def place_caches(rows_total, rows, k, v):
    """Device K/V caches [rows_total][Hkv][D], zero except the given rows."""
    hkv, d = k.shape[1], k.shape[2]
    kc = torch.zeros((rows_total, hkv, d), dtype=torch.int16, device=DEV)
    vc = torch.zeros_like(kc)
    idx = torch.from_numpy(np.asarray(rows, np.int64)).to(DEV)
    kc[idx] = dev(k)
    vc[idx] = dev(v)
    return kc, vc


CHUNK_MAX, CHUNK_MIN = 2048, 256   # positions per workgroup of the kernel
RESCALE_LOG2 = 8.0    # growth of the running maximum that triggers a rescale


def tolerance(qh, kr, vr, n, scale):
    """First-order fp32 error bound of one request's output (see the module docstring).
    qh: [Hq][D] float; kr, vr: [m][Hkv][D] float (the request's readable rows); n: its
    context length."""
    hq, hkv = qh.shape[0], kr.shape[1]
    g = hq // hkv
    kmax = np.sqrt((kr.astype(np.float64) ** 2).sum(axis=2)).max(axis=0)  # [Hkv]
    vmax = np.abs(vr).max(axis=(0, 2)).astype(np.float64)                # [Hkv]
    qn = np.sqrt((qh.astype(np.float64) ** 2).sum(axis=1))               # [Hq]
    heads = np.arange(hq) // g
    big_s = np.log2(np.e) * abs(scale) * qn * kmax[heads]
    rescales = 1 + np.ceil(2 * big_s / RESCALE_LOG2)
    chunks = -(-int(n) // CHUNK_MIN)
    return U * vmax[heads] * (CHUNK_MAX / 2 + 6 * rescales + 2 * chunks + 60 +
                              score_coefficient(g) * big_s)


def score_coefficient(group):
    """Weight of S in the bounds: 20 for the vector path's q.k (1 or 2 query heads per
    key/value head), 190 for the matrix-core path (4 or 8; see the module docstring)."""
    return 190 if group >= 4 else 20


def check(gpu, q, slots, rows, k, v, ctx_eff, sel, hq, hkv, scale, tag, exact=False):
    """Compare gpu[sel] with the oracle; rows/k/v hold the cache rows the requests read.
    exact: K is 0 and V integer-valued, so out * n must round to the oracle's sum exactly."""
    orc = oracle.get()
    order = np.argsort(rows)
    rows_s = np.asarray(rows, np.int64)[order]
    local = []
    for r in sel:
        s = slots[r]
        idx = np.full(len(s), -1, np.int64)
        ok = s >= 0
        if ok.any():
            j = np.searchsorted(rows_s, s[ok])
            assert (j < len(rows_s)).all() and (rows_s[j] == s[ok]).all(), "a read row is not drawn"
            idx[ok] = order[j]
        local.append(idx)
    want = orc.decode_attention(q, k, v, local, np.asarray(sel, np.int32), hq, hkv, scale)
    ratio = 0.0
    for i, r in enumerate(sel):
        got = gpu[r]
        assert np.isfinite(got).all(), f"{tag}: request {r} has non-finite output"
        idx = local[i][local[i] >= 0]
        if len(idx) == 0:
            assert (got == 0).all(), f"{tag}: request {r} reads nothing but is not 0"
            continue
        if exact:
            n = len(idx)
            g_sum = np.rint(got.astype(np.float64) * n)
            o_sum = np.rint(want[i] * n)
            assert np.abs(want[i] * n - o_sum).max() < 1e-6       # the oracle's sums are integers
            bad = np.argwhere(g_sum != o_sum)
            assert len(bad) == 0, f"{tag}: request {r}: {len(bad)} sums differ, first {bad[:3]}"
            continue
        tol = tolerance(f32(q[r]), f32(k[idx]), f32(v[idx]), ctx_eff[r], scale)
        err = np.abs(got.astype(np.float64) - want[i]).max(axis=1)
        worst = int(np.argmax(err / tol))
        assert (err <= tol).all(), (f"{tag}: request {r} head {worst}: error {err[worst]:.3e} "
                                    f"over the bound {tol[worst]:.3e}")
        ratio = max(ratio, float(err[worst] / tol[worst]))
    say(f"[decode] {tag}: largest error is {ratio:.3f} of the bound")


def parity(w, mode, hq, seed, lay=None, ctx_given=None, max_context=None, scale=None, sel=None,
           draw_rows=None, kind="normal", chunk=0):
    """Decode over layout `lay` (default: w's) with fresh q/K/V; check outputs and flags."""
    lay = lay or Layout(w)
    hkv = w.num_kv_heads
    ctx_w = np.array([rq.end for rq in w.requests] + [0] * (w.num_reqs - len(w.requests)),
                     np.int64)
    ctx_given = ctx_w if ctx_given is None else np.asarray(ctx_given, np.int64)
    if max_context is None:
        max_context = int(max(ctx_given.max(initial=0), 0))
    ctx_eff = np.clip(ctx_given, 0, max_context)
    count_flag = FLAG_COUNT if (ctx_eff != ctx_given).any() else 0
    slots, flags = expected_slots(lay, mode, ctx_eff)
    sel = list(range(w.num_reqs)) if sel is None else list(sel)
    if draw_rows is None:  # every row of the pool
        rows = None
    else:
        rows = np.unique(np.concatenate([slots[r][slots[r] >= 0] for r in sel] +
                                        [np.zeros(0, np.int64)]))
    q, _, rows, k, v = decode_inputs(w, hq, seed, rows=rows if rows is not None else
                                     np.arange(lay.rows, dtype=np.int64), kind=kind)
    scale = float(scale if scale is not None else w.head_dim ** -0.5)
    say(f"[decode] {w.name} {mode} Hq {hq} Hkv {hkv} bs {lay.bs} reqs {w.num_reqs} "
        f"max_context {max_context} checked {len(sel)} rows {len(rows)} scale {scale:.4f} "
        f"inputs {kind} chunk {chunk or 'auto'}")
    kc, vc = place_caches(lay.rows, rows, k, v)
    gpu, gflag = run_gpu(mode, lay, q, ctx_given, max_context, kc, vc, scale=scale, chunk=chunk)
    assert gflag == flags | count_flag, f"flags {gflag} != {flags | count_flag}"
    check(gpu, q, slots, rows, k, v, ctx_eff, sel, hq, hkv, scale, f"{w.name}/{mode}",
          exact=kind == "integers")
    return gpu, slots


# ---------------------------------------------------------------------------
# small workloads: ragged contexts around the 256-position chunk, every head grouping
# ---------------------------------------------------------------------------
def _dec(name, seed, contexts, bs, runs, hkv, pool, dummies=0, **kw):
    reqs = [Request(int(c), 1 if c else 0) for c in contexts]
    return custom(name, seed, reqs, block_size=bs, num_blocks=pool, runs=runs, num_kv_heads=hkv,
                  dummy_reqs=dummies, **kw)


def small_decodes():
    rng = np.random.Generator(np.random.PCG64([4711, 0]))
    return [
        # (workload, query heads)
        (_dec("ragged_g4", 1, [1, 255, 256, 257, 700, 1500, 3000, 4097, 0], 16,
              ("count", 1, 6), 8, 1200, dummies=2), 32),
        (_dec("bs32_g8", 2, rng.integers(1, 2000, 12), 32, ("count", 1, 4), 4, 1024), 32),
        (_dec("bs64_g1_16heads", 3, [63, 64, 65, 1000, 2049], 64, ("len", 1, 3), 16, 128), 16),
        (_dec("bs16_g2", 4, rng.integers(1, 1200, 9), 16, ("len", 1, 8), 2, 900), 4),
        (_dec("one_head", 5, [1, 2, 300, 513], 16, ("count", 1, 3), 1, 128), 1),
        (_dec("g8_one_kv_head", 6, [17, 600, 1025], 16, ("count", 2, 5), 1, 160), 8),
        # one block per run: the search over range_cum spans many entries
        (_dec("many_runs", 7, [3000, 4000, 257], 16, ("len", 1, 1), 8, 600,
              range_stride=300), 32),
        # block size 1: a chunk's 256 positions fall in 256 different runs
        (_dec("bs1_many_runs", 8, [600, 1100, 5], 1, ("len", 1, 1), 4, 2000,
              range_stride=1200), 16),
        # 64 query heads: over 8 key/value heads (8 per head, 8 waves) and over 16 (4 per head,
        # 16 waves)
        (_dec("hq64_g8", 10, [1, 700, 1300, 2100], 16, ("count", 1, 3), 8, 400), 64),
        (_dec("hq64_g4_16heads", 11, [513, 1025, 90], 32, ("count", 1, 3), 16, 120), 64),
        # 40 query heads over 5 key/value heads (G = 8): a chunk's heads split over two
        # workgroups of three waves, the second with one wave idle
        (_dec("hq40_g8_5heads", 13, [300, 1100, 2100, 17], 16, ("count", 1, 3), 5, 400), 40),
        # 6 query heads over 3 key/value heads: the combine's last group of four heads is partial
        (_dec("hq6_g2_3heads", 12, [40, 900, 1800, 2500], 16, ("count", 1, 3), 3, 500), 6),
        # 40 requests (a work list orders the chunks): empty ones, exact chunk multiples, tails
        (_dec("plan_40_reqs", 9, list(rng.integers(0, 2200, 34)) + [0, 256, 512, 1024, 2048, 1],
              16, ("count", 1, 4), 8, 6000, dummies=3), 32),
    ]


SMALL = small_decodes()
PLAN_CASE = SMALL[-1]


@pytest.mark.parametrize("mode", ["paged", "ranges"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: c[0].name)
def test_decode_small(case, mode):
    w, hq = case
    parity(w, mode, hq, seed=100 + len(w.name))
    parity(w, mode, hq, seed=200 + len(w.name), kind="integers")


@pytest.mark.parametrize("chunk", [256, 512, 1024, 2048])
@pytest.mark.parametrize("mode", ["paged", "ranges"])
def test_decode_chunk_lengths(mode, chunk):
    """Every chunk length the kernel takes, on contexts around its multiples."""
    w, hq = SMALL[0]
    parity(w, mode, hq, seed=20 + chunk, chunk=chunk)
    parity(w, mode, hq, seed=21 + chunk, chunk=chunk, kind="integers")
    w, hq = SMALL[2]
    parity(w, mode, hq, seed=22 + chunk, chunk=chunk)
    w, hq = PLAN_CASE
    parity(w, mode, hq, seed=23 + chunk, chunk=chunk)
    parity(w, mode, hq, seed=24 + chunk, chunk=chunk, kind="integers")


def test_decode_scale_and_longer_max_context():
    w, hq = SMALL[0]
    for mode in ("paged", "ranges"):
        parity(w, mode, hq, seed=3, scale=0.3, max_context=5000)   # chunks past every context
        parity(w, mode, hq, seed=4, scale=1.0)


@pytest.mark.parametrize("case", [0, -1], ids=["direct", "work_list"])
@pytest.mark.parametrize("mode", ["paged", "ranges"])
def test_decode_context_clamped(mode, case):
    """Lengths above max_context or negative are clamped (KVW_FLAG_COUNT)."""
    w, hq = SMALL[case]
    ctx = np.array([rq.end for rq in w.requests] + [0] * (w.num_reqs - len(w.requests)), np.int64)
    ctx[3] = 99999          # past max_context: clamped to it
    ctx[len(w.requests) - 1] = -7   # negative: no position, output 0
    ctx[len(w.requests)] = 300      # a dummy request with no blocks: every position is unmapped
    parity(w, mode, hq, seed=5, ctx_given=ctx, max_context=2000)


@pytest.mark.parametrize("mode", ["paged", "ranges"])
def test_decode_unmapped_tail(mode):
    """Positions past a request's blocks or ranges are skipped (whole chunks may be empty);
    counts above the stride are clamped with KVW_FLAG_COUNT."""
    w, hq = SMALL[0]
    nbpr = w.num_blocks_per_req.copy()
    nr = w.num_ranges.copy()
    nbpr[4], nbpr[6], nbpr[7] = 5, 0, w.table_stride + 3
    nr[4], nr[6], nr[7] = 1, 0, w.range_stride + 3
    lay = Layout(w, nbpr=nbpr, nr=nr)
    parity(w, mode, hq, seed=6, lay=lay)


def test_decode_bad_blocks():
    """A negative block id is skipped with KVW_FLAG_BAD_BLOCK; a block past the pool with
    KVW_FLAG_SLOT_OOB."""
    w, hq = SMALL[0]
    table = w.block_table.copy()
    table[5, 3] = -4
    table[6, 1] = w.num_blocks + 2
    parity(w, "paged", hq, seed=7, lay=Layout(w, table=table))
    rs = w.range_start.copy()
    rs[6, 0] = w.num_blocks + 10
    parity(w, "ranges", hq, seed=8, lay=Layout(w, rs=rs))


def test_decode_empty():
    w, hq = SMALL[0]
    lay = Layout(w)
    q, _, rows, k, v = decode_inputs(w, hq, 9, rows=np.arange(lay.rows, dtype=np.int64))
    kc, vc = place_caches(lay.rows, rows, k, v)
    ctx = np.array([rq.end for rq in w.requests] + [0, 0], np.int64)
    for mode in ("paged", "ranges"):
        gpu, flag = run_gpu(mode, lay, q, np.zeros_like(ctx), 0, kc, vc)
        assert flag == 0 and (gpu == 0).all()
        gpu, flag = run_gpu(mode, lay, q, ctx, 0, kc, vc)   # every length clamped to 0
        assert flag == FLAG_COUNT and (gpu == 0).all()
    out = torch.full((0, hq, 128), 1.0, dtype=torch.float32, device=DEV)
    kvw.kvw_decode_attention(mode=kvw.KVW_SLOTS_PAGED, q=dev(q[:0]), k_cache=kc, v_cache=vc,
                             context_lens=dev(ctx[:0].astype(np.int32)), max_context=100,
                             num_blocks=lay.num_blocks, block_size=lay.bs, out=out,
                             block_table=dev(lay.table), num_blocks_per_req=dev(lay.nbpr))
    torch.cuda.synchronize()


@pytest.mark.parametrize("hq", [8, 32], ids=["vector", "matrix_core"])
def test_decode_cache_without_rows(hq):
    """num_blocks = 0 with positions to attend: every slot lies past the cache, so every
    position is skipped with KVW_FLAG_SLOT_OOB and every output is exactly 0; no chunk holds a
    position, so none reads the cache (the matrix-core kernel's first-tile load included).  The
    cache pointers still point at a valid allocation, as the call requires."""
    w, _ = SMALL[0]
    lay = Layout(w, num_blocks=0)
    q = decode_inputs(w, hq, 10, rows=np.zeros(0, np.int64))[0]
    ctx = np.array([rq.end for rq in w.requests] + [0] * (w.num_reqs - len(w.requests)), np.int64)
    slots, flags = expected_slots(lay, "paged", ctx)
    assert flags == FLAG_SLOT_OOB and all((s < 0).all() for s in slots)
    kc = torch.zeros((16, w.num_kv_heads, w.head_dim), dtype=torch.int16, device=DEV)
    for mode in ("paged", "ranges"):
        gpu, flag = run_gpu(mode, lay, q, ctx, int(ctx.max()), kc, kc)
        assert flag == FLAG_SLOT_OOB and (gpu == 0).all()


def test_decode_reads_what_the_write_wrote():
    """One step end to end: kv_write stores each decode token's K/V, then decode attention reads
    the cache; the oracle does the same with its own write."""
    orc = oracle.get()
    w, hq = SMALL[0]
    lay = Layout(w)
    q, ctx, rows, k, v = decode_inputs(w, hq, 10, rows=np.arange(lay.rows, dtype=np.int64))
    kc, vc = place_caches(lay.rows, rows, k, v)
    key_h, value_h = w.kv_layer(0, 0), w.kv_layer(1, 0)
    slots_w, _ = orc.slot_mapping_ranges(w.query_start_loc, w.num_reqs, w.positions,
                                         w.max_num_tokens, w.range_start, w.range_len,
                                         w.range_cum, w.num_ranges, w.block_size)
    hkv = w.num_kv_heads
    kh = k.reshape(lay.rows, hkv * 128).copy()
    vh = v.reshape(lay.rows, hkv * 128).copy()
    orc.kv_write(slots_w, key_h[None], value_h[None], w.num_blocks, w.block_size, kh, vh)
    slot_out = torch.empty(w.max_num_tokens, dtype=torch.int64, device=DEV)
    kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_RANGES, query_start_loc=dev(w.query_start_loc),
                     num_reqs=w.num_reqs, positions=dev(w.positions),
                     max_num_tokens=w.max_num_tokens, range_start=dev(w.range_start),
                     range_len=dev(w.range_len), range_cum=dev(w.range_cum),
                     num_ranges=dev(w.num_ranges), block_size=w.block_size,
                     num_blocks=w.num_blocks,
                     key=dev(key_h).view(1, w.max_num_tokens, hkv, 128),
                     value=dev(value_h).view(1, w.max_num_tokens, hkv, 128),
                     k_cache=kc, v_cache=vc, slot_mapping_out=slot_out)
    gpu, flag = run_gpu("ranges", lay, q, ctx, int(ctx.max()), kc, vc)
    assert flag == 0
    slots, _ = expected_slots(lay, "ranges", ctx)
    check(gpu, q, slots, rows, kh.reshape(lay.rows, hkv, 128), vh.reshape(lay.rows, hkv, 128),
          ctx, list(range(w.num_reqs)), hq, hkv, w.head_dim ** -0.5, "after write")


# ---------------------------------------------------------------------------
# full sizes: sampled requests against the oracle, the rest by a property
# ---------------------------------------------------------------------------
def full_size(w, lay, hq, sel, seed, kind="normal"):
    """Both modes on the full workload; only the rows that `sel` reads hold drawn K/V.  Every
    other request that reads none of them sees zeros and must give exactly 0 (an oversubscribed
    pool shares history blocks between requests; those are only checked to be finite)."""
    outs = []
    for mode in ("paged", "ranges"):
        gpu, slots = parity(w, mode, hq, seed, lay=lay, sel=sel, draw_rows=True, kind=kind)
        drawn = np.unique(np.concatenate([slots[r][slots[r] >= 0] for r in sel]))
        zero = 0
        for r in range(w.num_reqs):
            if r in sel:
                continue
            assert np.isfinite(gpu[r]).all()
            if not np.isin(slots[r], drawn).any():
                assert (gpu[r] == 0).all(), f"request {r} reads only zeros but is not 0"
                zero += 1
        say(f"[decode] {zero} of {w.num_reqs - len(sel)} unsampled requests read only zeros")
        assert zero > 0
        outs.append(gpu)
    # the two resolutions give the same slots, so the same arithmetic and the same bits
    assert np.array_equal(outs[0], outs[1])


def test_decode_step_full():
    """256 decodes with context U[1, 8192], Llama-3-8B heads (32 query / 8 key-value)."""
    w = config("decode_step")
    full_size(w, Layout(w), 32, sel=[0, 17, 100, 201, 255], seed=11)
    full_size(w, Layout(w), 32, sel=[5, 64, 130, 250], seed=13, kind="integers")


@pytest.mark.parametrize("r", [1, 4096])
def test_decode_long_context_full(r):
    """16 requests at 128K context, 32 query / 8 key-value heads, manager block size 32."""
    w = long_context(r)
    full_size(w, Layout(w), 32, sel=[3 + r % 11], seed=12)
    full_size(w, Layout(w), 32, sel=[9 + r % 5], seed=14, kind="integers")


def test_decode_long_context_full_64_heads():
    """16 requests at 128K context with 64 query heads over the 8 key-value heads (G = 8, a
    70B-class shape): each chunk's heads go to two workgroups, at full size."""
    w = long_context(4096)
    full_size(w, Layout(w), 64, sel=[6], seed=15)
    full_size(w, Layout(w), 64, sel=[12], seed=16, kind="integers")


# ---------------------------------------------------------------------------
# graph capture: launch shapes depend only on num_reqs, max_context and strides
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["paged", "ranges"])
def test_decode_graph_replay(mode):
    """Captured once at a padded request count and max_context, replayed with three batches of
    other lengths, layouts and queries (inputs refilled eagerly between replays).  Every replay
    equals an eager call bit for bit, and the oracle within the bound."""
    reqs, max_ctx, pool, bs, hkv, hq, stride, rstride = 10, 3000, 2400, 16, 8, 32, 188, 8

    def batch(seed):
        rng = np.random.Generator(np.random.PCG64([seed, 3]))
        n = int(rng.integers(5, reqs + 1))
        return _dec(f"graph_{seed}", seed, rng.integers(1, max_ctx + 1, n), bs, ("count", 1, 5),
                    hkv, pool, dummies=reqs - n, table_stride=stride, range_stride=rstride)

    batches = [batch(4900 + i) for i in range(3)]
    rows = pool * bs
    q_s = torch.empty((reqs, hq, 128), dtype=torch.int16, device=DEV)
    ctx_s = torch.empty(reqs, dtype=torch.int32, device=DEV)
    maps = {"block_table": torch.empty((reqs, stride), dtype=torch.int32, device=DEV),
            "num_blocks_per_req": torch.empty(reqs, dtype=torch.int32, device=DEV),
            "range_start": torch.empty((reqs, rstride), dtype=torch.int32, device=DEV),
            "range_len": torch.empty((reqs, rstride), dtype=torch.int32, device=DEV),
            "range_cum": torch.empty((reqs, rstride), dtype=torch.int32, device=DEV),
            "num_ranges": torch.empty(reqs, dtype=torch.int32, device=DEV)}
    kc = torch.empty((rows, hkv, 128), dtype=torch.int16, device=DEV)
    vc = torch.empty_like(kc)
    out = torch.empty((reqs, hq, 128), dtype=torch.float32, device=DEV)
    out_eager = torch.empty_like(out)
    ws = torch.empty(kvw.kvw_decode_workspace_size(reqs, max_ctx, hq), dtype=torch.uint8,
                     device=DEV)
    flag = new_flag()
    used = (("block_table", "num_blocks_per_req") if mode == "paged" else
            ("range_start", "range_len", "range_cum", "num_ranges"))
    kind = kvw.KVW_SLOTS_PAGED if mode == "paged" else kvw.KVW_SLOTS_RANGES

    def call(o):
        kvw.kvw_decode_attention(mode=kind, q=q_s, k_cache=kc, v_cache=vc, context_lens=ctx_s,
                                 max_context=max_ctx, num_blocks=pool, block_size=bs, out=o,
                                 workspace=ws, err_flag=flag, **{k: maps[k] for k in used})

    def load(w, seed):
        q, ctx, _, k, v = decode_inputs(w, hq, seed, rows=np.arange(rows, dtype=np.int64))
        q_s.copy_(dev(q))
        ctx_s.copy_(dev(ctx))
        kc.copy_(dev(k))
        vc.copy_(dev(v))
        for name in used:
            maps[name].copy_(dev(getattr(w, name)))
        flag.zero_()
        return q, ctx, k, v

    load(batches[0], 1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out)
    torch.cuda.synchronize()

    for rep, w in enumerate(batches + batches[:1]):
        say(f"[decode graph] {mode} replay {rep}: {w.describe()}")
        q, ctx, k, v = load(w, 10 + rep)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host(out)
        assert int(flag.item()) == 0
        call(out_eager)
        torch.cuda.synchronize()
        assert np.array_equal(got, host(out_eager)), "replay differs from the eager call"
        slots, _ = expected_slots(Layout(w), mode, ctx.astype(np.int64))
        check(got, q, slots, np.arange(rows, dtype=np.int64), k, v, ctx, list(range(reqs)), hq,
              hkv, 128 ** -0.5, f"graph {mode} replay {rep}")


def test_decode_through_the_written_table():
    """The whole step, then the read: kv_write (ranges, manager block size 32) stores the step's
    K/V and, in its slot-mapping launch, the attention side's table at kernel block size 16;
    decode attention then reads the cache through that table (paged, bs 16) and through the
    manager's range descriptors (ranges, bs 32).  Same slots, so the two outputs are equal bit
    for bit, and both match the oracle."""
    orc = oracle.get()
    reqs = [Request(e, n) for e, n in ((700, 40), (1500, 1), (2048, 300), (33, 33), (1025, 7))]
    w = custom("step_then_read", 4990, reqs, block_size=32, num_blocks=300, runs=("count", 1, 4),
               kernel_block_size=16, dummy_reqs=2)
    hq, hkv, k = 32, w.num_kv_heads, w.blocks_per_kv_block
    rows = w.num_blocks * w.block_size
    q, ctx, _, kh, vh = decode_inputs(w, hq, 77, rows=np.arange(rows, dtype=np.int64))
    kc, vc = place_caches(rows, np.arange(rows, dtype=np.int64), kh, vh)
    key_h, value_h = w.kv_layer(0, 0), w.kv_layer(1, 0)
    width = w.table_stride * k
    table = torch.full((w.num_reqs, width), -5, dtype=torch.int32, device=DEV)
    counts = torch.full((w.num_reqs,), -5, dtype=torch.int32, device=DEV)
    flag = new_flag()
    kvw.kvw_kv_write(mode=kvw.KVW_SLOTS_RANGES, query_start_loc=dev(w.query_start_loc),
                     num_reqs=w.num_reqs, positions=dev(w.positions),
                     max_num_tokens=w.max_num_tokens, range_start=dev(w.range_start),
                     range_len=dev(w.range_len), range_cum=dev(w.range_cum),
                     num_ranges=dev(w.num_ranges), block_size=w.block_size,
                     num_blocks=w.num_blocks,
                     key=dev(key_h).view(1, w.max_num_tokens, hkv, 128),
                     value=dev(value_h).view(1, w.max_num_tokens, hkv, 128),
                     k_cache=kc, v_cache=vc,
                     slot_mapping_out=torch.empty(w.max_num_tokens, dtype=torch.int64, device=DEV),
                     table_out=table, table_counts_out=counts, table_block_size=16, err_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    # the oracle's cache after its own write of the same step
    slots_w, _ = orc.slot_mapping_ranges(w.query_start_loc, w.num_reqs, w.positions,
                                         w.max_num_tokens, w.range_start, w.range_len,
                                         w.range_cum, w.num_ranges, w.block_size)
    ek = kh.reshape(rows, hkv * 128).copy()
    ev = vh.reshape(rows, hkv * 128).copy()
    orc.kv_write(slots_w, key_h[None], value_h[None], w.num_blocks, w.block_size, ek, ev)
    # read through the written kernel-unit table (paged, bs 16) and the manager's ranges (bs 32)
    lay16 = Layout(w, block_size=16, num_blocks=w.num_blocks * k, table=host(table),
                   nbpr=host(counts))
    got16, f16 = run_gpu("paged", lay16, q, ctx, int(ctx.max()), kc, vc)
    got32, f32_ = run_gpu("ranges", Layout(w), q, ctx, int(ctx.max()), kc, vc)
    assert f16 == 0 and f32_ == 0
    assert np.array_equal(got16, got32), "the two resolutions differ"
    slots, _ = expected_slots(Layout(w), "ranges", ctx.astype(np.int64))
    slots16, _ = expected_slots(lay16, "paged", ctx.astype(np.int64))
    assert all(np.array_equal(a, b) for a, b in zip(slots, slots16))
    check(got16, q, slots, np.arange(rows, dtype=np.int64), ek.reshape(rows, hkv, 128),
          ev.reshape(rows, hkv, 128), ctx, list(range(w.num_reqs)), hq, hkv, 128 ** -0.5,
          "through the written table")


# ---------------------------------------------------------------------------
# decode context parallelism: each rank attends its own positions; log-sum-exp merge
# ---------------------------------------------------------------------------
def lse_tolerance(qh, kr, n, scale, lse):
    """Bound on |lse error| per query head, from the same summation structure as `tolerance`:
    the normalizer's relative error plus the score error, plus the final rounding."""
    hq, hkv = qh.shape[0], kr.shape[1]
    g = hq // hkv
    kmax = np.sqrt((kr.astype(np.float64) ** 2).sum(axis=2)).max(axis=0)
    qn = np.sqrt((qh.astype(np.float64) ** 2).sum(axis=1))
    big_s = np.log2(np.e) * abs(scale) * qn * kmax[np.arange(hq) // g]
    rescales = 1 + np.ceil(2 * big_s / RESCALE_LOG2)
    chunks = -(-int(n) // CHUNK_MIN)
    return U * (CHUNK_MAX / 2 + 6 * rescales + 2 * chunks + 60 + score_coefficient(g) * big_s +
                np.abs(lse))


@pytest.mark.parametrize("world,inter", [(1, 1), (2, 1), (2, 16), (3, 4), (4, 8)])
@pytest.mark.parametrize("mode", ["paged", "ranges"])
def test_decode_context_parallel(mode, world, inter):
    """Each rank attends the positions it holds, from its own cache (block_size slots per block,
    the write's context-parallel placement), and reports its log-sum-exp; kvw_decode_merge of the
    ranks' results equals attention over every position.  Every rank is also checked alone."""
    orc = oracle.get()
    reqs = [Request(e, 1 if e else 0) for e in (1, 300, 1000, 2500, 40, 0, 777)]
    w = custom("cp_read", 4995, reqs, block_size=16, num_blocks=700, runs=("count", 1, 4),
               dummy_reqs=1)
    hq, hkv, bs, scale = 32, w.num_kv_heads, w.block_size, 128 ** -0.5
    ctx = np.array([rq.end for rq in w.requests] + [0], np.int64)
    total = int(ctx.sum())
    first = np.concatenate([[0], np.cumsum(ctx)[:-1]])       # flat index of each request's position 0
    q, _, _, k_flat, v_flat = decode_inputs(w, hq, 31, rows=np.arange(total, dtype=np.int64))
    # the oracle's attention over every position: flat rows, slot = flat index
    flat_slots = [np.arange(first[r], first[r] + ctx[r], dtype=np.int64) for r in range(w.num_reqs)]
    want, want_lse = orc.decode_attention(q, k_flat, v_flat, flat_slots, np.arange(w.num_reqs),
                                          hq, hkv, scale, with_lse=True)
    qsl = np.zeros(w.num_reqs + 1, np.int32)
    qsl[1:] = np.cumsum(ctx)
    pos = np.concatenate([np.arange(c, dtype=np.int64) for c in ctx])
    rows = w.num_blocks * bs
    outs = torch.empty((world, w.num_reqs, hq, 128), dtype=torch.float32, device=DEV)
    lses = torch.empty((world, w.num_reqs, hq), dtype=torch.float32, device=DEV)
    qd, cl = dev(q), dev(ctx.astype(np.int32))
    for rank in range(world):
        # this rank's slots (-1 for the other ranks' positions), from the oracle
        if mode == "paged":
            sl, fl = orc.slot_mapping_paged_cp(qsl, w.num_reqs, pos, total, w.block_table,
                                               w.num_blocks_per_req, bs, world, rank, inter)
        else:
            sl, fl = orc.slot_mapping_ranges_cp(qsl, w.num_reqs, pos, total, w.range_start,
                                                w.range_len, w.range_cum, w.num_ranges, bs, world,
                                                rank, inter)
        assert fl == 0
        held = sl >= 0
        kr = np.zeros((rows, hkv, 128), np.uint16)
        vr = np.zeros_like(kr)
        kr[sl[held]] = k_flat[held]          # position t of the flat order sits at its slot
        vr[sl[held]] = v_flat[held]
        kc, vc = dev(kr), dev(vr)
        flag = new_flag()
        common = dict(q=qd, k_cache=kc, v_cache=vc, context_lens=cl, max_context=int(ctx.max()),
                      num_blocks=w.num_blocks, block_size=bs, out=outs[rank], err_flag=flag,
                      cp_world_size=world, cp_rank=rank, cp_interleave_size=inter,
                      lse_out=lses[rank])
        if mode == "paged":
            kvw.kvw_decode_attention(mode=kvw.KVW_SLOTS_PAGED, block_table=dev(w.block_table),
                                     num_blocks_per_req=dev(w.num_blocks_per_req), **common)
        else:
            kvw.kvw_decode_attention(mode=kvw.KVW_SLOTS_RANGES, range_start=dev(w.range_start),
                                     range_len=dev(w.range_len), range_cum=dev(w.range_cum),
                                     num_ranges=dev(w.num_ranges), **common)
        torch.cuda.synchronize()
        assert int(flag.item()) == 0
        # the rank alone: attention over the positions it holds
        rank_slots = [sl[qsl[r]:qsl[r + 1]] for r in range(w.num_reqs)]
        say(f"[decode cp] {mode} W={world} I={inter} rank {rank}: {int(held.sum())} of {total}")
        got = host(outs[rank])
        check(got, q, rank_slots, np.arange(rows, dtype=np.int64), kr, vr, ctx,
              list(range(w.num_reqs)), hq, hkv, scale, f"cp {mode} W={world} rank {rank}")
        o_r, l_r = orc.decode_attention(q, kr, vr, rank_slots, np.arange(w.num_reqs), hq, hkv,
                                        scale, with_lse=True)
        g_l = host(lses[rank]).astype(np.float64)
        for r in range(w.num_reqs):
            mine = rank_slots[r][rank_slots[r] >= 0]
            if len(mine) == 0:
                assert np.all(g_l[r] == -np.inf)
                continue
            tol = lse_tolerance(f32(q[r]), f32(kr[mine]), ctx[r], scale, l_r[r])
            assert np.all(np.abs(g_l[r] - l_r[r]) <= tol), f"rank {rank} request {r}: lse"
    # the merge of the ranks' results against attention over every position
    merged = torch.full((w.num_reqs, hq, 128), float("nan"), dtype=torch.float32, device=DEV)
    merged_lse = torch.full((w.num_reqs, hq), float("nan"), dtype=torch.float32, device=DEV)
    kvw.kvw_decode_merge(outs, lses, merged, merged_lse)
    torch.cuda.synchronize()
    got = host(merged).astype(np.float64)
    got_lse = host(merged_lse).astype(np.float64)
    ratio = 0.0
    for r in range(w.num_reqs):
        if ctx[r] == 0:
            assert (got[r] == 0).all() and np.all(got_lse[r] == -np.inf)
            continue
        rows_r = flat_slots[r]
        tol = tolerance(f32(q[r]), f32(k_flat[rows_r]), f32(v_flat[rows_r]), ctx[r], scale)
        err = np.abs(got[r] - want[r]).max(axis=1)
        assert (err <= tol).all(), f"merged request {r}: error {err.max():.3e}"
        ltol = lse_tolerance(f32(q[r]), f32(k_flat[rows_r]), ctx[r], scale, want_lse[r])
        assert np.all(np.abs(got_lse[r] - want_lse[r]) <= ltol), f"merged request {r}: lse"
        ratio = max(ratio, float((err / tol).max()))
    say(f"[decode cp] {mode} W={world} I={inter}: merged, largest error {ratio:.3f} of the bound")
    if world == 1:  # one part: the merge returns it
        assert np.array_equal(host(merged), host(outs[0]))
