"""Speculative flash-decode step of attention-level speculation (ALSpec) on
AMD Instinct MI355X (gfx950).

The work runs in hand-written HIP kernels behind the C ABI of
include/alspec.h (libalspec.so, built in-tree); this package is the thin
Python binding over it.  Importing fails if the library is not built.
"""
from ._binding import (AlspecError, Events, Handle, KV_BF16, KV_F32,
                       LAYERS_WS_RING, LIB_PATH, NOALLOC_SCRATCH_BYTES,
                       POST_MAX_BATCH,
                       Params, PostParams, PostWeights, alloc_outputs, alloc_post_workspace,
                       alloc_workspace, make_post_params, post_attention,
                       post_weights_struct, post_workspace_size,
                       flash_decode_exact, last_error, lse_combine,
                       make_params,
                       order_after_verify, params_for, plan_splits,
                       sink_approx, spec_decode, spec_decode_layers,
                       spec_decode_noalloc,
                       status_string, verify, version, workspace_size)

__all__ = ["AlspecError", "Events", "Handle", "KV_BF16", "KV_F32",
           "LAYERS_WS_RING", "LIB_PATH", "NOALLOC_SCRATCH_BYTES",
           "POST_MAX_BATCH", "Params",
           "PostParams",
           "PostWeights", "alloc_outputs", "alloc_post_workspace",
           "alloc_workspace", "make_post_params", "post_attention",
           "post_weights_struct", "post_workspace_size",
           "flash_decode_exact", "last_error", "lse_combine", "make_params",
           "order_after_verify", "params_for",
           "plan_splits", "sink_approx", "spec_decode",
           "spec_decode_layers", "spec_decode_noalloc", "status_string",
           "verify", "version", "workspace_size"]
