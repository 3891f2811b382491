"""Independent oracle computations (one per head, or per group of query tiles
of one head) in worker processes on the host, so that the full-size parity
tests of the long clip and the packed sequence finish in minutes.

Test infrastructure: the workers import only the oracle, the seeded workload
description and numpy; they never touch the GPU.  Workers are spawned (not
forked from a process that has initialised the GPU) and each runs one BLAS
thread, so a pool of W workers uses W host cores.

Every task takes the natural-layout bf16 bit patterns of one head (int16
[N, D]) and builds the one-head oracle plan of that head's tile shape: the
oracle's tiling, budgets and selection of a head depend only on its shape and
the segments, so a one-head plan gives exactly that head's part of the
all-heads oracle.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
from typing import Callable, Iterable, List

import numpy as np


def workers() -> int:
    """Host cores the pool uses: at most 16 (a GPU machine's CPU share)."""
    return max(1, min(16, os.cpu_count() or 1))


def _init() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def pool_map(fn: Callable, items: Iterable, nworkers: int = 0) -> List:
    items = list(items)
    if not items:
        return []
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=nworkers or workers(), mp_context=ctx, initializer=_init) as ex:
        return list(ex.map(fn, items))


def _bf16_bits_to_f64(x: np.ndarray) -> np.ndarray:
    """int16 bf16 bit patterns -> fp64 values (exact)."""
    return (x.astype(np.int32).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _one_head_plan(spec):
    from oracle import veda_oracle as vo
    segments, head_dim, shape, budget_mode, keep_num, keep_den, fixed_k = spec
    return vo.Plan(segments, 1, head_dim, [tuple(shape)], budget_mode, keep_num, keep_den, fixed_k)


def head_spec(w, h: int, budget_mode=None):
    """Picklable description of head h's one-head oracle plan."""
    mode = w.budget_mode if budget_mode is None else budget_mode
    return (w.segments, w.head_dim, tuple(w.tile_shapes[h]), mode, w.keep_num, w.keep_den, w.fixed_k)


def front_task(args):
    """Oracle permute, pool, project, score and select of one head.

    args = (spec, q_bits [N, D] int16, k_bits [N, D] int16, w_q [D, 3D] fp32,
    w_k [D, 3D] fp32).  Returns (scores fp32 [n, n], row lengths int64 [n],
    concatenated ascending column lists int64)."""
    from oracle import veda_oracle as vo
    spec, qb, kb, wq, wk = args
    op = _one_head_plan(spec)
    qp = vo.permute_forward(op, _bf16_bits_to_f64(qb)[:, None, :])
    kp = vo.permute_forward(op, _bf16_bits_to_f64(kb)[:, None, :])
    qh = vo.project(op, vo.pool_tiles(op, qp), wq[None])
    kh = vo.project(op, vo.pool_tiles(op, kp), wk[None])
    scores = vo.score_pairs(op, qh, kh)
    sel = vo.select_blocks(op, scores)
    lens = np.array([len(r) for r in sel[0]], dtype=np.int64)
    return scores[0], lens, np.concatenate(sel[0]).astype(np.int64)


def attention_task(args):
    """Oracle attention (O10) of the listed query tiles of one head.

    args = (spec, q_bits, k_bits, v_bits (int16 [N, D] each), tiles (list of
    query tile indices), cols (list of the selected key tiles of each), scale).
    Returns a list of (O [valid, D] fp64, LSE [valid] fp64) per tile."""
    from oracle import veda_oracle as vo
    spec, qb, kb, vb_, tiles, cols, scale = args
    op = _one_head_plan(spec)
    qp = vo.permute_forward(op, _bf16_bits_to_f64(qb)[:, None, :])
    kp = vo.permute_forward(op, _bf16_bits_to_f64(kb)[:, None, :])
    vp = vo.permute_forward(op, _bf16_bits_to_f64(vb_)[:, None, :])
    return [vo.attention_row_tile(op, 0, i, qp, kp, vp, c, scale) for i, c in zip(tiles, cols)]


def dense_heat_task(args):
    """The oracle's dense LSE (O10 over every key tile) and block heat (O11)
    of one head.  args = (spec, q_bits, k_bits, scale).  Returns (LSE fp64
    [L_h] in permuted row order, NaN on padding rows; heat fp64 [n, n])."""
    from oracle import veda_oracle as vo
    spec, qb, kb, scale = args
    op = _one_head_plan(spec)
    qp = vo.permute_forward(op, _bf16_bits_to_f64(qb)[:, None, :])
    kp = vo.permute_forward(op, _bf16_bits_to_f64(kb)[:, None, :])
    _, L = vo.block_sparse_attention(op, qp, kp, kp, vo.all_blocks_selection(op), scale)
    heat = vo.block_heat(op, qp, kp, L, scale)[0]
    return L, heat


def chunks(seq, n: int):
    """Split seq into n nearly equal consecutive parts (empty parts dropped)."""
    seq = list(seq)
    k, r = divmod(len(seq), n)
    out, at = [], 0
    for c in range(n):
        m = k + (1 if c < r else 0)
        if m:
            out.append(seq[at:at + m])
        at += m
    return out
