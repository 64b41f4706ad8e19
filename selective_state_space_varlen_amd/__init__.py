"""Packed variable-length Mamba-1 sequence operators on MI355X (gfx950).

The operators are HIP kernels in libssmpack.so behind a C ABI
(include/ssmpack.h); this package is the thin Python binding over it plus a
pipeline helper that chains the calls of one Mamba block's sequence-wise part.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    PackPlan,
    SsmpError,
    conv1d_pack_bwd,
    conv1d_pack_bwd_states_workspace_bytes,
    conv1d_pack_bwd_workspace_bytes,
    conv1d_pack_fwd,
    load,
    selective_scan_pack_bwd,
    selective_scan_pack_bwd_ck,
    selective_scan_pack_bwd_scratch_bytes,
    selective_scan_pack_fwd,
    selective_scan_pack_fwd_ck,
    selective_scan_pack_fwd_noalloc,
    selective_scan_pack_fwd_scratch_bytes,
    selective_scan_pack_saved_bytes,
    selective_scan_pack_workspace_bytes,
    varlen_pack_indices,
    varlen_pack_plan,
)
from .pipeline import forward, backward  # noqa: F401
