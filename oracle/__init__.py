"""CPU fp64 oracle for tile-window 3D attention, pooled global attention and
the gated merge.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``video_dit_sparse_amd``) never imports it, and it never imports the product
path: the two share no code.
"""
from .ref import (  # noqa: F401
    token_coords,
    tile_index,
    tile_counts,
    tile_extent,
    window_radius,
    sta_mask_row,
    WINDOW_MODES,
    mode_tile_index,
    mode_tile_counts,
    window_tiles,
    mode_mask_row,
    sta_ref,
    dense_ref,
    attention_weights_ref,
    pool_ref,
    pooled_grid,
    global_ref,
    merge_ref,
    merge_lse_ref,
    union_attention_ref,
    upsample_bilinear_ref,
    compressed_global_ref,
    hier_pooled_ref,
    attention_bwd_ref,
    sta_bwd_ref,
    global_bwd_ref,
    sta_pair_count_ref,
    sta_flops_ref,
    global_flops_ref,
    dense_flops_ref,
    hier_pair_count_ref,
    to_f64,
)
