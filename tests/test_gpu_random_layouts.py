"""Seeded random layouts through the K/V write and decode attention (needs an MI355X).

Each case draws a batch from its seed: the request count, every request's context and
new-token lengths (empty requests included), the block size (1 to 64), how each request's
blocks split into runs, the pool's slack, one or two layers, the key/value head count,
padding rows past the real tokens and dummy requests.  It then runs the fused write in three
of its modes and decode attention over the same layout (paged and ranges, a query-head
grouping drawn too), each against the oracle with the checks of the hand-picked cases:
byte-exact slots and cache planes for the write; the derived fp32 bound, or the exact integer
sums for the integer input kind, for attention.  The hand-picked cases choose their shapes one
by one; these cover combinations nobody listed.
"""
from __future__ import annotations

import numpy as np
import pytest

from parity import say
from test_gpu_decode_attention import parity as decode_parity
from test_gpu_parity import WRITE_MODES, check_kv_write
from workloads import custom
from workloads.gen import Request

pytestmark = pytest.mark.gpu

SEEDS = list(range(24))


def random_case(seed: int):
    """(workload, write modes, query heads, decode input kind) drawn from the seed."""
    rng = np.random.Generator(np.random.PCG64([9100, seed]))
    bs = int(rng.choice([1, 2, 4, 8, 16, 32, 64]))
    n_req = int(rng.integers(1, 40))
    reqs = []
    for _ in range(n_req):
        end = int(rng.integers(0, 2500)) if rng.random() > 0.1 else 0
        n_new = int(rng.integers(0, end + 1)) if rng.random() < 0.5 else min(end, 1)
        reqs.append(Request(end, n_new))
    blocks = sum(-(-rq.end // bs) for rq in reqs)
    pool = int(blocks * rng.uniform(1.1, 2.0)) + 8
    runs = ("count", 1, int(rng.integers(1, 9))) if rng.random() < 0.5 else \
        ("len", 1, int(rng.integers(1, 65)))
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    n_tok = sum(rq.n_new for rq in reqs)
    w = custom(f"random_{seed}", 9100 + seed, reqs, block_size=bs, num_blocks=pool, runs=runs,
               num_layers=int(rng.integers(1, 3)), num_kv_heads=hkv, head_dim=128,
               max_num_tokens=n_tok + int(rng.integers(0, 40)),
               dummy_reqs=int(rng.integers(0, 4)))
    modes = [str(m) for m in rng.choice(WRITE_MODES, size=3, replace=False)]
    kind = "integers" if rng.random() < 0.3 else "normal"
    return w, modes, hkv * group, kind


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layout(seed):
    w, modes, hq, kind = random_case(seed)
    say(f"[random] seed {seed}: {w.describe()} write modes {modes} decode Hq {hq} {kind}")
    for mode in modes:
        check_kv_write(w, mode)
    for mode in ("paged", "ranges"):
        decode_parity(w, mode, hq, seed=9200 + seed, kind=kind)
