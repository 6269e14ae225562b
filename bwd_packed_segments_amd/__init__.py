"""MI355X (gfx950) fused attention forward and backward over packed segments.

The compute lives in ``libbps_attn.so`` (hand-written HIP behind a C ABI,
declared in ``include/bps_attn.h``).  The Python layer here only marshals
arguments: it allocates outputs and workspace with torch, passes raw device
pointers and the current HIP stream, and turns status codes into
exceptions.  Importing the package does not load the library; the first
call does, and it raises if the library is missing.
"""

from .binding import (  # noqa: F401
    ATTN_FORCE_GENERAL,
    ATTN_FUSED_BWD,
    ATTN_LOG_ROUTE,
    ATTN_REVERSE_SCHEDULE,
    ATTN_BWD_ALL,
    ATTN_BWD_DKDV,
    ATTN_BWD_DQ,
    ATTN_BWD_PREPARE,
    AttnError,
    BwdPlan,
    FwdPlan,
    Segments,
    attn_bwd,
    attn_bwd_noalloc,
    attn_bwd_ex,
    attn_debug_mask,
    attn_fwd,
    attn_fwd_ex,
    attn_ring_bwd,
    attn_ring_fwd,
    bwd_workspace_size,
    fwd_workspace_size,
    lib,
    library_path,
    route_counts,
    validate_fwd,
)
