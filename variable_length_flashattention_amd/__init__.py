"""MI355X (gfx950) variable-length FlashAttention: forward (packed or paged
K/V, grouped-query), backward, and paged GQA decode (one-shot or stateful).

The compute lives in ``librra.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/rra.h``).  This package is a thin ctypes binding over it;
torch supplies device memory and streams only.
"""
from .binding import (  # noqa: F401
    RraError,
    library_path,
    load_library,
    rra_status_string,
    rra_varlen_attn_fwd,
    rra_varlen_attn_fwd_gqa,
    rra_varlen_attn_fwd_paged,
    rra_varlen_attn_bwd,
    rra_varlen_attn_bwd_workspace_bytes,
    rra_varlen_block_q,
    rra_paged_decode_attn,
    rra_paged_decode_workspace_bytes,
    rra_paged_decode_attn_noalloc,
    rra_paged_decode_scratch_bytes,
    rra_paged_decode_state_init,
    rra_paged_decode_step,
    rra_paged_decode_finalize,
    rra_pack_rows,
    rra_unpack_rows,
    rra_debug_varlen_tile_map,
    rra_debug_paged_gather,
    varlen_attn_fwd,
    varlen_attn_fwd_paged,
    varlen_attn_bwd,
    paged_decode_attn,
    decode_state_init,
    paged_decode_step,
    paged_decode_finalize,
    pack_padded,
    unpack_to_padded,
)
