"""The allocator model against hand-worked sequences and recomputed invariants (CPU)."""
import pytest

import alloc_pins as AP
from oracle.range_alloc import RangeAllocOracle


def make(num_blocks, alignment, first_block, rows):
    return RangeAllocOracle(num_blocks, alignment, first_block, rows)


def test_golden_sequences():
    AP.pin_golden(make)


def test_lone_growth_keeps_one_range():
    AP.pin_lone_growth(make)


@pytest.mark.parametrize("seed", range(8))
def test_random_sequences(seed):
    AP.pin_random(make, seeds=[seed])
