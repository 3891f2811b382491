"""Veda block-sparse attention for AMD Instinct MI355X (gfx950).

The compute path is libveda.so (hand-written HIP kernels behind the C ABI in
include/veda.h); this package only builds it and binds it with ctypes.
"""

from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, Plan, VedaError, lib, veda_abi_version, veda_available, veda_block_heat, veda_mask_mass, veda_output_error, veda_tile_plan_vote, veda_mask_transpose,
    veda_block_sparse_attn_bwd,
    veda_block_sparse_attn_fwd, veda_last_error, veda_permute_tiles, veda_plan_copy_budgets, veda_score_tiles_noalloc,
    veda_plan_copy_perm, veda_plan_copy_row_ptr, veda_plan_copy_valid, veda_plan_create,
    veda_plan_destroy, veda_plan_head, veda_plan_query, veda_plan_upload, veda_score_tiles,
    veda_permute_qkv, veda_score_pooled, VEDA_LAYOUT_NATURAL, VEDA_LAYOUT_PERMUTED,
    veda_select_blocks, VEDA_BUDGET_ALL, VEDA_BUDGET_FIXED_K, VEDA_BUDGET_KEEP_RATIO,
    VEDA_PERMUTE_FORWARD, VEDA_PERMUTE_FORWARD_TRANSPOSED, VEDA_PERMUTE_INVERSE, VEDA_SEG_DENSE1D,
    VEDA_SEG_VIDEO3D)
