"""MI355X-native local-window attention: the local Softmax branch of VDN-H3
hybrid video attention (forward and backward), the complement linear branch
and the two-branch fusion (separately, or in the softmax branch's epilogue),
as hand-written HIP for gfx950 behind a C ABI.

The HIP library is loaded lazily on the first call (see binding.lib()); there
is no CPU fallback.
"""

from .binding import (  # noqa: F401
    VDN_BF16,
    VDN_FP8_E4M3,
    VdnError,
    lib,
    hybrid_attn_fwd,
    hybrid_fuse,
    linear_branch_fwd,
    local_attn_bwd,
    local_attn_fwd,
    vdn_hybrid_attn_fwd,
    vdn_hybrid_attn_workspace_bytes,
    vdn_hybrid_fuse,
    vdn_last_error,
    vdn_linear_branch_fwd,
    vdn_linear_branch_workspace_bytes,
    vdn_local_attn_count_pairs,
    vdn_local_attn_bwd,
    vdn_local_attn_fwd,
    vdn_local_attn_kernel_tile_m,
    vdn_local_attn_key_blocks,
    vdn_local_attn_key_intervals,
    vdn_local_attn_num_query_blocks,
    vdn_local_attn_tile_schedule,
)
