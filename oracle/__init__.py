"""CPU fp64 oracle (test infrastructure only; see reference.py's header)."""

from .reference import (  # noqa: F401
    to_f64,
    attention,
    merge,
    merge_many,
    updated_positions,
    update_count,
    gate_count,
    head_cosine,
    gate_cosine,
    kl_rows,
    lock_update,
    varlen_pack,
    step_gates,
    refresh_steps,
    prefix_rows,
    block_keys,
    prefix_rows_in_blocks,
    block_rows,
    run_block,
    run_varlen,
)
