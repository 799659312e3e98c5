"""kvw_decode_attention_noalloc (the decode-attention entry point that allocates nothing: its
workspace is a static per-GPU array) against kvw_decode_attention with a caller-owned workspace,
through the C-ABI (needs an MI355X).

Both run the same kernels on the same inputs, so outputs, log-sum-exps and flag words must agree
bit for bit.  Two calls in a row, the second with a smaller batch, so the second runs over what
the first left in the shared array: the 256-request decode step (32 query heads over 8 key/value
heads, 34 MB of workspace with its work list), then six requests of 20,480 positions over one
range per 16 blocks (8 MB, no work list).  Cache contents are seeded N(0, 1) bf16 drawn on the
device: the comparison is between two entry points, not against the oracle (kvw_decode_attention
itself is checked against the oracle elsewhere).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_46_amd as kvw
from parity import DEV, dev, new_flag, say
from workloads import config, long_context

pytestmark = pytest.mark.gpu

HQ = 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvw.library()
    yield
    torch.cuda.synchronize()


def _inputs(w, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    rows = w.num_blocks * w.block_size
    shape = (rows, w.num_kv_heads, w.head_dim)
    kc = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    vc = torch.randn(shape, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((w.num_reqs, HQ, w.head_dim), generator=gen, device=DEV,
                    dtype=torch.float32).to(torch.bfloat16)
    ctx = np.array([rq.end for rq in w.requests] + [0] * (w.num_reqs - len(w.requests)), np.int32)
    return q, kc, vc, ctx


def _call(fn, w, mode, q, kc, vc, ctx, workspace=None):
    out = torch.full((w.num_reqs, HQ, w.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((w.num_reqs, HQ), float("nan"), dtype=torch.float32, device=DEV)
    flag = new_flag()
    kw = dict(q=q, k_cache=kc, v_cache=vc, context_lens=dev(ctx), max_context=int(ctx.max()),
              num_blocks=w.num_blocks, block_size=w.block_size, out=out, err_flag=flag,
              lse_out=lse)
    if workspace is not None:
        kw["workspace"] = workspace
    if mode == "paged":
        fn(mode=kvw.KVW_SLOTS_PAGED, block_table=dev(w.block_table),
           num_blocks_per_req=dev(w.num_blocks_per_req), **kw)
    else:
        fn(mode=kvw.KVW_SLOTS_RANGES, range_start=dev(w.range_start), range_len=dev(w.range_len),
           range_cum=dev(w.range_cum), num_ranges=dev(w.num_ranges), **kw)
    torch.cuda.synchronize()
    return out, lse, int(flag.item())


@pytest.mark.parametrize("mode", ["paged", "ranges"])
def test_noalloc_matches_the_workspace_entry_point(mode):
    small = long_context(16, seed=4750, num_reqs=6, context=20480, chunk=1)
    for step, (w, seed) in enumerate(((config("decode_step"), 4751), (small, 4752))):
        say(f"[noalloc] call {step + 1}: {w.describe()} {mode}")
        q, kc, vc, ctx = _inputs(w, seed)
        need = kvw.kvw_decode_workspace_size(w.num_reqs, int(ctx.max()), HQ, w.head_dim)
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        ref = _call(kvw.kvw_decode_attention, w, mode, q, kc, vc, ctx, workspace=ws)
        got = _call(kvw.kvw_decode_attention_noalloc, w, mode, q, kc, vc, ctx)
        assert torch.isfinite(ref[0]).all() and torch.isfinite(got[0]).all()
        assert torch.equal(got[0].view(torch.int32), ref[0].view(torch.int32)), "outputs differ"
        assert torch.equal(got[1].view(torch.int32), ref[1].view(torch.int32)), "lse differ"
        assert got[2] == ref[2] == 0
        del kc, vc, ws
        torch.cuda.empty_cache()
