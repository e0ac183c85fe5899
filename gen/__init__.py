"""Seeded synthetic inputs for the sparse-delta-memory decode step and token gather.

This package draws inputs only: banks, slot lists, weights, values, gates and
chunk lengths, and the compact-stash position map a caller derives from them. It holds none of the method's arithmetic, and both the oracle
side and the HIP side of every test and benchmark take their inputs from it.
"""

from .workloads import (  # noqa: F401
    DecodeWorkload,
    GatherWorkload,
    WORKLOADS,
    compact_positions,
    decode_bank,
    decode_step_inputs,
    decode_sequence,
    gather_bank,
    gather_inputs,
    live_tokens,
    sub_seed,
)
