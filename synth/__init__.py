"""Seeded synthetic inputs for paged decode attention.

This package only draws inputs: context lengths, the order in which physical
block ids are handed out, and the q / K / V values. It holds none of the
method's arithmetic (no paging, no attention, no quantisation), so both the
CPU oracle and the HIP path can be fed from it without sharing code.
"""
from .workloads import (  # noqa: F401
    DecodeWorkload,
    PrefixWorkload,
    tiny_decode,
    gqa_decode,
    long_context,
    prefix_sharing,
    mixed_lengths,
    random_case,
    blocks_needed_for_pool,
)
