"""MI355X-native (gfx950) AttnRes depth-aggregation hot path.

The product is libattnres.so, a C-ABI library of hand-written HIP kernels
(include/attnres.h); ``binding`` is its thin Python binding.
"""
from .binding import (  # noqa: F401
    ATTNRES_BF16, ATTNRES_F32, AttnResError, NativeSublayer, attnres_aggregate,
    attnres_atomic_block_size, attnres_block_layout, attnres_block_stack_forward,
    attnres_phase1_batched, attnres_phase2_merge, attnres_stack_workspace_bytes,
    attnres_timing_enable, attnres_timing_read, attnres_timing_reset,
)
