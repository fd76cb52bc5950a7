"""Seeded synthetic inputs for block-diffusion cached split attention.

This package only draws random numbers and lays them out; it computes no
attention, no merge, no gate decision and no packing.  Both the CPU oracle's
tests and the GPU path's tests and benchmark take their inputs from here.
"""

from .synth import (  # noqa: F401
    BlockSchedule,
    VarlenBatch,
    bf16_bits_to_f32,
    round_to_bf16_bits,
    make_block_schedule,
    make_key_block_lists,
    make_logit_pair,
    make_varlen_batch,
    preset,
    PRESETS,
)
