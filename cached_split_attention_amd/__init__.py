"""Cached split attention for block diffusion on MI355X (gfx950).

The compute lives in libba.so (HIP kernels behind the C-ABI of include/ba.h);
this package is its Python binding.  Importing it requires the built library:
there is no CPU fallback.
"""

from ._lib import BaError, lib  # noqa: F401
from .api import (  # noqa: F401
    BA_GATE_COUNT,
    BA_GATE_COSINE,
    BA_GATE_COUNT_CUM,
    BA_GATE_ROWS,
    ba_block_attn,
    ba_gated_split_attn,
    ba_gated_split_attn_gate_workspace,
    ba_kl_lock,
    ba_lse_merge,
    ba_prefix_attn,
    ba_prefix_attn_merge,
    ba_prefix_attn_noalloc,
    ba_prefix_attn_rows,
    ba_prefix_attn_workspace,
    ba_reuse_gate,
    ba_reuse_gate_workspace,
    ba_sparse_prefix_attn,
    ba_sparse_prefix_attn_workspace,
    ba_split_attn,
    ba_varlen_pack,
    ba_version,
)
from .step import CachedBlockAttention  # noqa: F401

lib()  # fail loudly at import if the HIP library is missing
