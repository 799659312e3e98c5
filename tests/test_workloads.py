"""The seeded input generator: determinism and the layout invariants it promises."""
import numpy as np
import pytest

from workloads import BF16_MARKER_ONE, CONFIG_NAMES, config, long_context, small_cases


def _check_layout(w):
    R = w.num_reqs
    qsl = w.query_start_loc
    assert qsl[0] == 0 and (np.diff(qsl) >= 0).all() and qsl[-1] <= w.max_num_tokens
    for r in range(w.max_num_reqs):
        nb = int(w.num_blocks_per_req[r])
        row = w.block_table[r, :nb]
        assert (row >= 1).all() and (row < w.num_blocks).all(), "block 0 handed out or id past pool"
        assert (w.block_table[r, nb:] == 0).all()
        n = int(w.num_ranges[r])
        st, ln, cm = w.range_start[r, :n], w.range_len[r, :n], w.range_cum[r, :n]
        assert (ln >= 1).all()
        assert (cm == np.concatenate([[0], np.cumsum(ln)[:-1]])).all() if n else True
        # the row is the concatenation of the runs
        cat = np.concatenate([np.arange(s, s + l) for s, l in zip(st, ln)]) if n else np.zeros(0)
        assert np.array_equal(cat, row)
    # positions of each request are its last n_new positions
    for r, rq in enumerate(w.requests):
        p = w.positions[qsl[r]:qsl[r + 1]]
        assert np.array_equal(p, np.arange(rq.end - rq.n_new, rq.end))


def _written_blocks(w):
    """(request, block id) of every block holding a token scheduled this step."""
    out = []
    qsl = w.query_start_loc
    for r in range(len(w.requests)):
        nb = int(w.num_blocks_per_req[r])
        lb = w.positions[qsl[r]:qsl[r + 1]] // w.block_size
        lb = lb[lb < nb]
        out += [(r, int(b)) for b in np.unique(w.block_table[r, lb])]
    return out


@pytest.mark.parametrize("w", small_cases(), ids=lambda w: w.name)
def test_small_layouts(w):
    _check_layout(w)


@pytest.mark.parametrize("name", ["tiny_prefill", "decode_step", "mixed_chunked", "full_32_layer"])
def test_study_layouts(name):
    w = config(name)
    _check_layout(w)
    wb = _written_blocks(w)
    ids = [b for _, b in wb]
    assert len(ids) == len(set(ids)), "a written block is shared"
    # a written block is never aliased by any other block of the pool layout
    every = np.concatenate([w.block_table[r, :w.num_blocks_per_req[r]]
                            for r in range(len(w.requests))])
    counts = np.bincount(every, minlength=w.num_blocks)
    assert (counts[ids] == 1).all()


@pytest.mark.parametrize("r", [1, 16, 512, 4096])
def test_long_context_layout(r):
    w = long_context(r)
    _check_layout(w)
    assert (w.num_ranges == r).all()
    every = w.block_table.ravel()
    assert len(np.unique(every)) == every.size == w.num_blocks - 1


def test_study_sizes():
    w = config("tiny_prefill")
    assert w.query_start_loc.tolist() == [0, 7, 40, 140, 390] and w.max_num_tokens == 512
    w = config("decode_step")
    assert w.num_reqs == 256 and w.num_tokens == 256 and w.num_blocks == 65536
    w = config("mixed_chunked")
    assert w.num_reqs == 64 and w.num_tokens == 8192
    assert sorted(rq.n_new for rq in w.requests)[-8:][0] >= 512
    assert sum(1 for rq in w.requests if rq.n_new > 1) == 8
    w = long_context(4096)
    assert (w.num_tokens, w.block_size, w.kernel_block_size) == (131072, 32, 16)
    w = config("full_32_layer")
    assert (w.num_reqs, w.num_tokens, w.num_layers, w.num_blocks) == (512, 16384, 32, 32768)
    assert sum(1 for rq in w.requests if rq.n_new == 125) == 128


def test_determinism_and_kv():
    a, b = config("tiny_prefill"), config("tiny_prefill")
    for f in ("query_start_loc", "positions", "block_table", "range_start", "range_len"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    k = a.kv_layer(0, 0)
    assert np.array_equal(k, b.kv_layer(0, 0))
    assert not np.array_equal(k, a.kv_layer(1, 0))
    assert (k[a.num_tokens:] == BF16_MARKER_ONE).all()
    real = k[:a.num_tokens].view(np.uint16).astype(np.uint32) << 16
    vals = real.view(np.float32)
    assert np.isfinite(vals).all() and abs(vals.mean()) < 0.05 and abs(vals.std() - 1) < 0.05


def test_config_names():
    assert CONFIG_NAMES == ("tiny_prefill", "decode_step", "mixed_chunked", "long_context",
                            "full_32_layer")
