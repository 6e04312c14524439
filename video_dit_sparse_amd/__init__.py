"""Tile-window sparse attention for video latents on MI355X (gfx950).

Python face of libvdsa.so: the three calls of the hot path
(``sta_attn_fwd``, ``global_pooled_attn_fwd``, ``dual_branch_merge``), the global
branch on the library's static scratch for callers that cannot allocate
(``global_pooled_attn_fwd_noalloc``), the
exact log-sum-exp merge (``dual_branch_merge_lse``), the global branch with
either merge fused into it (``global_pooled_attn_merge_fwd``), the pooling
step alone (``kv_avgpool_fwd``), UltraGen's hierarchical and compressed
global variants (``hier_pooled_attn_fwd``, ``compressed_global_attn_fwd``),
the backward passes (``sta_attn_bwd``,
``global_pooled_attn_bwd``) and the effective-work counters.  The
sliding-tile calls take a ``window_mode`` ("clip", "inward", "cyclic").
"""
from ._lib import (  # noqa: F401
    WINDOW_MODES,
    VdsaError,
    abi_version,
    compressed_global_attn_fwd,
    dual_branch_merge,
    dual_branch_merge_lse,
    compressed_global_flops,
    global_flops,
    hier_flops,
    global_pooled_attn_fwd,
    global_pooled_attn_fwd_noalloc,
    global_pooled_attn_merge_fwd,
    global_pooled_attn_bwd,
    global_pooled_attn_bwd_workspace_size,
    global_pooled_attn_workspace_size,
    hier_pooled_attn_fwd,
    kv_avgpool_fwd,
    lib,
    sta_attn_fwd,
    sta_attn_bwd,
    sta_attn_bwd_workspace_size,
    sta_flops,
    sta_kernel_name,
)
