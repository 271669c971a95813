"""chunked_causal_linear_amd - chunkwise-parallel causal linear attention on MI355X.

The compute path is ``liblinattn.so`` (hand-written HIP for gfx950) behind the
C ABI in ``include/la.h``; ``binding`` marshals torch tensors into it.  The
library is loaded on first use; calling any entry point without it raises
``LibraryNotBuilt``.
"""
from .binding import (  # noqa: F401
    EXPORTS, FMAPS, LAError, LibraryNotBuilt, Forward, chunk_output, chunk_states, chunked_forward, feature_map,
    forward_group, forward_workspace_bytes, lib, recurrent_step, state_scan, loglinear_forward, loglinear_levels,
    LogLinearForward, DeltaForward, delta_forward, delta_chunk_transform, recurrent_step_delta,
    recurrent_step_loglinear, loglinear_prefix_levels, recurrent_step_i8,
    chunked_forward_noalloc,
)

__all__ = ["chunked_forward", "Forward", "chunk_states", "chunk_output", "state_scan", "feature_map", "recurrent_step",
           "forward_workspace_bytes", "lib", "LAError", "LibraryNotBuilt", "EXPORTS", "FMAPS", "loglinear_forward",
           "loglinear_levels", "LogLinearForward", "DeltaForward", "delta_forward", "delta_chunk_transform",
           "recurrent_step_delta", "chunked_forward_noalloc", "recurrent_step_loglinear",
           "loglinear_prefix_levels", "recurrent_step_i8"]
