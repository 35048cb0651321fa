"""MI355X-native retention operator: chunkwise and parallel forward, backward, decode step, gated
variants, and the gated retention layer around it.

The operator runs in libretention_fwd.so (hand-written HIP kernels for gfx950) behind
the C ABI in include/retention.h; this package is its Python binding.  Importing the
package does not load the library; the first call does, and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    RetentionError,
    bwd_workspace_bytes,
    calib_mfma,
    gated_msr_fwd,
    gated_retention_chunkwise_bwd,
    gated_retention_chunkwise_fwd,
    gated_retention_decode_step,
    gated_retention_parallel_fwd,
    lib,
    msr_workspace_bytes,
    profile_enable,
    profile_read,
    retention_chunkwise_bwd,
    retention_chunkwise_fwd,
    retention_chunkwise_fwd_noalloc,
    retention_decode_step,
    retention_parallel_fwd,
    workspace_bytes,
)

__all__ = [
    "retention_chunkwise_fwd",
    "retention_chunkwise_bwd",
    "gated_retention_chunkwise_bwd",
    "bwd_workspace_bytes",
    "gated_retention_chunkwise_fwd",
    "retention_decode_step",
    "gated_retention_decode_step",
    "retention_parallel_fwd",
    "gated_retention_parallel_fwd",
    "workspace_bytes",
    "gated_msr_fwd",
    "msr_workspace_bytes",
    "RetentionError",
    "lib",
    "profile_enable",
    "profile_read",
    "calib_mfma",
    "retention_chunkwise_fwd_noalloc",
]
