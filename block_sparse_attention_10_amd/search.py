"""Tile-plan search on the GPU (Miowtion project page, Key Features: oracle
tile-plan search by relative output MSE under the best mask, majority vote,
at most two shapes per layer).

For every sample (q, k, v of one layer) the dense output in natural token
order is computed once (all-blocks attention under the first candidate's
tiling; in natural order it does not depend on the tiling).  Then for every
candidate (t, h, w) tile shape, through libveda:
  permute (veda_permute_qkv) -> the dense LSE and the block heat in one pass
  (veda_dense_lse_heat) -> oracle mask (veda_select_blocks on the heat, the
  layer's budgets) -> block-sparse attention over it -> relative output
  error per head against the dense output (veda_output_error);
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

    def plans(shape):
        shapes = [tuple(shape)] * num_heads
        p = vb.Plan(segments, num_heads, head_dim, shapes, budget_mode, keep_num, keep_den, fixed_k)
        pd = vb.Plan(segments, num_heads, head_dim, shapes, vb.VEDA_BUDGET_ALL)
        pairs = p.info["total_pairs"]
        d_rp = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
        d_col = torch.empty(pd.info["nnz"], dtype=torch.int32, device=dev)
        pd.select(torch.zeros(pairs, dtype=torch.float32, device=dev), d_rp, d_col, stream=stream)
        return p, pd, d_rp, d_col

    # dense outputs, natural order, one per sample
    p, pd, d_rp, d_col = plans(candidates[0])
    qp, kp, vt, ws = p.empty_perm(), p.empty_perm(), p.empty_vt(), p.empty_workspace()
    o_dense = []
    for q, k, v in samples:
        o = torch.empty_like(q)
        p.permute_qkv(q, k, v, qp, kp, vt, ws, stream=stream)
        pd.attention(qp, kp, vt, d_rp, d_col, scale, o, stream=stream, o_layout=vb.VEDA_LAYOUT_NATURAL)
        o_dense.append(o)
    for ci, shape in enumerate(candidates):
        p, pd, d_rp, d_col = plans(shape)
        qp, kp, vt, ws = p.empty_perm(), p.empty_perm(), p.empty_vt(), p.empty_workspace()
        heat = torch.empty(p.info["total_pairs"], dtype=torch.float32, device=dev)
        heat_ws = torch.empty(pd.info["heat_workspace_bytes"] // 4, dtype=torch.float32, device=dev)
        rp = torch.empty(p.T + 1, dtype=torch.int32, device=dev)
        col = torch.empty(p.info["nnz"], dtype=torch.int32, device=dev)
        lse = torch.empty(p.R, dtype=torch.float32, device=dev)
        for si, (q, k, v) in enumerate(samples):
            o_sparse = torch.empty_like(q)
            p.permute_qkv(q, k, v, qp, kp, vt, ws, stream=stream)
            pd.lse_heat(qp, kp, d_rp, d_col, scale, lse, heat, heat_ws, stream=stream)
            p.select(heat, rp, col, stream=stream)
            p.attention(qp, kp, vt, rp, col, scale, o_sparse, stream=stream, o_layout=vb.VEDA_LAYOUT_NATURAL)
            p.output_error(o_sparse, o_dense[si], err[si, ci], stream=stream)
    torch.cuda.synchronize()
    err_h = err.cpu().numpy()
    return err_h, vb.veda_tile_plan_vote(err_h, max_shapes)
