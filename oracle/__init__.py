"""fp64 CPU oracle for variable-length attention and paged GQA decode.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the GPU library never does.  See ``oracle.c`` for the
definitions and the page sections they follow.
"""
from .oracle import (  # noqa: F401
    build,
    load,
    varlen_attn,
    varlen_attn_rows,
    varlen_attn_paged,
    varlen_attn_bwd,
    paged_decode,
    paged_decode_recurrent,
    decode_state_init,
    paged_decode_step,
    paged_decode_finalize,
    paged_gather,
    varlen_tile_map,
    default_threads,
)
