"""The CPU oracle against facts outside itself (no GPU needed)."""
import numpy as np
import pytest

import oracle
import oracle_pins as P
from workloads import config, long_context, small_cases

MiB = 1 << 20


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(scope="module")
def small():
    return small_cases()


def light(ws, limit=40 * MiB):
    return [w for w in ws
            if w.num_layers * w.num_blocks * w.block_size * w.bytes_per_token <= limit]


def test_golden_slot_values_bs16(orc):
    P.pin_golden_bs16(orc)


def test_golden_figure6_sequence_bs4(orc):
    P.pin_figure6(orc)


def test_token_at_a_time_allocation(orc):
    P.pin_fill_simulation(orc, seeds=range(24))


def test_exhaustive_tiny_layouts(orc):
    P.pin_enumeration(orc)


def test_padding_rules(orc):
    P.pin_padding_rules(orc)


def test_range_equals_gather_small(orc, small):
    P.pin_range_equals_gather(orc, small)


@pytest.mark.parametrize("name", ["tiny_prefill", "decode_step", "mixed_chunked", "full_32_layer"])
def test_range_equals_gather_study_configs(orc, name):
    P.pin_range_equals_gather(orc, [config(name)])


@pytest.mark.parametrize("r", [1, 16, 512, 4096])
def test_range_equals_gather_long_context(orc, r):
    """128K context: manager-unit ranges at bs 32 == expanded table at bs 16."""
    w = long_context(r)
    P.pin_range_equals_gather(orc, [w])
    k = w.blocks_per_kv_block
    kt, f = orc.map_to_kernel_blocks(w.block_table, w.num_blocks_per_req, w.block_size,
                                     w.kernel_block_size)
    assert f == 0
    sk, _ = orc.slot_mapping_paged(w.query_start_loc, w.num_reqs, w.positions, w.max_num_tokens,
                                   kt, w.num_blocks_per_req * k, w.kernel_block_size)
    sr, _ = orc.slot_mapping_ranges(w.query_start_loc, w.num_reqs, w.positions, w.max_num_tokens,
                                    w.range_start, w.range_len, w.range_cum, w.num_ranges,
                                    w.block_size)
    assert np.array_equal(sk, sr)
    assert (sk >= 0).all() and len(np.unique(sk)) == len(sk)


def test_expansion(orc):
    P.pin_expansion(orc)


def test_table_fill(orc, small):
    P.pin_table_fill(orc, small + [config(n) for n in ("tiny_prefill", "decode_step",
                                                       "mixed_chunked")])


@pytest.mark.parametrize("r", [1, 4096])
def test_table_fill_long_context(orc, r):
    """128K context: manager runs filled at kernel block size == the expanded manager table."""
    w = long_context(r)
    k = w.blocks_per_kv_block
    kt, _ = orc.map_to_kernel_blocks(w.block_table, w.num_blocks_per_req, w.block_size,
                                     w.kernel_block_size)
    out, cnt, f = orc.ranges_to_block_table(w.range_start, w.range_len, w.range_cum, w.num_ranges,
                                            w.block_size, w.kernel_block_size, w.table_stride * k)
    assert f == 0 and np.array_equal(out, kt) and np.array_equal(cnt, w.num_blocks_per_req * k)


def test_context_parallel(orc, small):
    P.pin_context_parallel(orc, small)


def test_decode_attention(orc):
    P.pin_attention(orc)


def test_coordinate_form(orc):
    P.pin_coordinates(orc)


def test_kv_write(orc, small):
    P.pin_kv_write(orc, light(small))


def test_oracle_rejects_bad_inputs(orc):
    qsl = np.array([0, 3, 2], np.int32)
    with pytest.raises(oracle.OracleError):
        orc.slot_mapping_paged(qsl, 2, np.zeros(3, np.int64), 3, np.zeros((2, 1), np.int32),
                               None, 16)
    qsl = np.array([0, 2], np.int32)
    st = np.array([[4, 9]], np.int32)
    ln = np.array([[1, 1]], np.int32)
    bad_cum = np.array([[0, 2]], np.int32)
    with pytest.raises(oracle.OracleError):
        orc.slot_mapping_ranges(qsl, 1, np.zeros(2, np.int64), 2, st, ln, bad_cum,
                                np.array([2], np.int32), 16)
    key = np.zeros((1, 2, 8), np.uint16)
    win = np.zeros((4, 8), np.uint16)
    with pytest.raises(oracle.OracleError):
        orc.kv_write(np.array([1, 1]), key, key, 2, 2, win, win.copy())
