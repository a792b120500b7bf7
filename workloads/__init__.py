"""Seeded synthetic inputs for paged decode attention.

This package only draws random numbers and lays them out: context lengths,
block-table assignments, q / K / V values and poisoned (unused) cache slots.
It contains none of the attention arithmetic, so both the CPU oracle and the
GPU path can consume exactly the same bits from it without sharing any of the
method's code.
"""

from .synth import (  # noqa: F401
    BLOCK_SIZE,
    CONFIGS,
    DecodeCase,
    ReplaySchedule,
    bf16_bits,
    block_refcounts,
    build_case,
    chunked_prefill_case,
    config_case,
    decode_step_inputs,
    fork_case,
    fork_groups,
    parallel_normal,
    replay_schedule,
    replay_step_values,
)
