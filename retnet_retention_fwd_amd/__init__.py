"""MI355X-native retention operator: chunkwise forward and backward, decode step, gated variants.

The operator runs in libretention_fwd.so (hand-written HIP kernels for gfx950) behind
the C ABI in include/retention.h; this package is its Python binding.  Importing the
package does not load the library; the first call does, and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    RetentionError,
    bwd_workspace_bytes,
    gated_retention_chunkwise_bwd,
    gated_retention_chunkwise_fwd,
    gated_retention_decode_step,
    lib,
    profile_enable,
    profile_read,
    retention_chunkwise_bwd,
    retention_chunkwise_fwd,
    retention_decode_step,
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
    "workspace_bytes",
    "RetentionError",
    "lib",
    "profile_enable",
    "profile_read",
]
