"""Tile-plan search on the GPU (Miowtion project page, Key Features: oracle
tile-plan search by relative output MSE under the best mask, majority vote,
at most two shapes per layer).

For every sample (q, k, v of one layer) and every candidate (t, h, w) tile
shape, run through libveda:
  permute (veda_permute_qkv) -> all-blocks attention (dense output in natural
  order and the dense LSE) -> block heat (veda_block_heat) -> oracle mask
  (veda_select_blocks on the heat, the layer's budgets) -> block-sparse
  attention over it -> relative output error per head (veda_output_error);
then the vote over the error table (veda_tile_plan_vote).  This module only
sequences library calls and owns the device buffers (torch allocations).
"""

from . import binding as vb


def tile_plan_search(segments, num_heads, head_dim, candidates, budget_mode, keep_num, keep_den, fixed_k,
                     samples, scale, max_shapes=2, stream=None):
    """samples: list of (q, k, v) CUDA bf16 tensors [N, H, D].
    Returns (err, choice): err host float64 [samples, candidates, heads],
    choice host int32 [heads] (candidate index of every head)."""
    import torch
    S, C = len(samples), len(candidates)
    dev = "cuda"
    err = torch.empty((S, C, num_heads), dtype=torch.float64, device=dev)
    for ci, shape in enumerate(candidates):
        shapes = [tuple(shape)] * num_heads
        p = vb.Plan(segments, num_heads, head_dim, shapes, budget_mode, keep_num, keep_den, fixed_k)
        pd = vb.Plan(segments, num_heads, head_dim, shapes, vb.VEDA_BUDGET_ALL)
        qp, kp, vt, ws = p.empty_perm(), p.empty_perm(), p.empty_vt(), p.empty_workspace()
        pairs = p.info["total_pairs"]
        heat = torch.empty(pairs, dtype=torch.float32, device=dev)
        d_rp = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
        d_col = torch.empty(pd.info["nnz"], dtype=torch.int32, device=dev)
        pd.select(torch.zeros(pairs, dtype=torch.float32, device=dev), d_rp, d_col, stream=stream)
        rp = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
        col = torch.empty(p.info["nnz"], dtype=torch.int32, device=dev)
        lse = torch.empty(p.R, dtype=torch.float32, device=dev)
        for si, (q, k, v) in enumerate(samples):
            o_dense = torch.empty_like(q)
            o_sparse = torch.empty_like(q)
            p.permute_qkv(q, k, v, qp, kp, vt, ws, stream=stream)
            pd.attention(qp, kp, vt, d_rp, d_col, scale, o_dense, lse, stream=stream,
                         o_layout=vb.VEDA_LAYOUT_NATURAL)
            p.heat(qp, kp, lse, scale, heat, stream=stream)
            p.select(heat, rp, col, stream=stream)
            p.attention(qp, kp, vt, rp, col, scale, o_sparse, stream=stream, o_layout=vb.VEDA_LAYOUT_NATURAL)
            p.output_error(o_sparse, o_dense, err[si, ci], stream=stream)
    torch.cuda.synchronize()
    err_h = err.cpu().numpy()
    return err_h, vb.veda_tile_plan_vote(err_h, max_shapes)
