"""Seeded synthetic inputs for the paged KV-cache write path.

This package only *draws* inputs: request lengths, positions, the physical
block layout of each request (as a block-table row and as contiguous runs)
and the K/V payload.  It computes no slot, no offset and no cache content;
those belong to the code under test and to the oracle, which both consume
these inputs unchanged.
"""
from .gen import (  # noqa: F401
    BF16_MARKER_ONE,
    BF16_SENTINEL,
    CONFIG_NAMES,
    Request,
    Workload,
    config,
    custom,
    decode_inputs,
    long_context,
    range_tables,
    small_cases,
)
