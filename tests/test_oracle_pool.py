"""The per-head oracle tasks of tests/oracle_pool (used by the full-size GPU
parity tests) give the all-heads oracle's results: one-head plans, bf16 bit
patterns decoded on the worker side, and the pool's chunking.  Scores and
selections are bit-exact; fp64 attention, LSE and heat agree to 1e-12
relative (a worker's one-thread BLAS sums in another order than a
multi-threaded one)."""

import numpy as np
import torch

import oracle_pool as opool
import veda_workloads as wl
from oracle import veda_oracle as vo


def _bits(x):
    return x.contiguous().view(torch.int16).numpy()


def _small():
    V = wl.VIDEO3D
    return wl.Workload(91, "small_packed_2shapes", (wl.Segment(V, (2, 8, 12), 0), wl.Segment(V, (4, 10, 12), 192),
                                                    wl.Segment(wl.DENSE1D, (1, 1, 200), 672)),
                       4, 128, ((2, 8, 8), (4, 4, 8), (2, 8, 8), (4, 4, 8)), wl.KEEP_RATIO, 1, 3)


def test_chunks():
    assert opool.chunks(range(10), 3) == [[0, 1, 2, 3], [4, 5, 6], [7, 8, 9]]
    assert opool.chunks(range(2), 5) == [[0], [1]]
    assert opool.chunks([], 4) == []


def test_bf16_bits_decode():
    x = torch.tensor([0.0, -0.0, 1.5, -2.75, 3.0e38, -1e-30], dtype=torch.float32).to(torch.bfloat16)
    got = opool._bf16_bits_to_f64(_bits(x))
    assert np.array_equal(got.view(np.uint64), x.to(torch.float64).numpy().view(np.uint64))


def test_tasks_equal_all_heads_oracle():
    w = _small()
    inp = wl.make_inputs(w, seed=w.index)
    op = vo.Plan.from_workload(w)
    ref = vo.run_path(op, inp["q"].double().numpy(), inp["k"].double().numpy(), inp["v"].double().numpy(),
                      inp["w_q"].numpy(), inp["w_k"].numpy(), w.softmax_scale)
    qb, kb, vb_ = _bits(inp["q"]), _bits(inp["k"]), _bits(inp["v"])
    fronts = opool.pool_map(opool.front_task, [
        (opool.head_spec(w, h), np.ascontiguousarray(qb[:, h]), np.ascontiguousarray(kb[:, h]),
         inp["w_q"].numpy()[h], inp["w_k"].numpy()[h]) for h in range(w.num_heads)], nworkers=2)
    for h, (scores, lens, cols) in enumerate(fronts):
        assert np.array_equal(scores.view(np.uint32), ref["scores"][h].view(np.uint32))
        assert np.array_equal(lens, [len(r) for r in ref["selection"][h]])
        assert np.array_equal(cols, np.concatenate(ref["selection"][h]))
    h = 1
    sel = ref["selection"][h]
    parts = opool.chunks(range(op.heads[h].num_tiles), 3)
    res = opool.pool_map(opool.attention_task, [
        (opool.head_spec(w, h), np.ascontiguousarray(qb[:, h]), np.ascontiguousarray(kb[:, h]),
         np.ascontiguousarray(vb_[:, h]), p, [sel[i] for i in p], w.softmax_scale) for p in parts], nworkers=2)
    for p, rr in zip(parts, res):
        for i, (O, L) in zip(p, rr):
            r0 = op.row_offset[h] + 128 * i
            nv = op.heads[h].tiles[i].valid
            assert np.allclose(O, ref["o_perm"][r0:r0 + nv], rtol=1e-12, atol=1e-14)
            assert np.allclose(L, ref["lse"][r0:r0 + nv], rtol=1e-12, atol=1e-14)


def test_dense_heat_task_equals_oracle():
    w = _small()
    inp = wl.make_inputs(w, seed=w.index)
    op = vo.Plan(w.segments, w.num_heads, w.head_dim, w.tile_shapes, wl.ALL_BLOCKS, 1, 1, 0)
    qp = vo.permute_forward(op, inp["q"].double().numpy())
    kp = vo.permute_forward(op, inp["k"].double().numpy())
    _, L = vo.block_sparse_attention(op, qp, kp, kp, vo.all_blocks_selection(op), w.softmax_scale)
    heat = vo.block_heat(op, qp, kp, L, w.softmax_scale)
    qb, kb = _bits(inp["q"]), _bits(inp["k"])
    res = opool.pool_map(opool.dense_heat_task, [
        (opool.head_spec(w, h, budget_mode=wl.ALL_BLOCKS), np.ascontiguousarray(qb[:, h]),
         np.ascontiguousarray(kb[:, h]), w.softmax_scale) for h in range(w.num_heads)], nworkers=2)
    for h, (Lh, hh) in enumerate(res):
        r0 = op.row_offset[h]
        assert np.array_equal(np.isnan(Lh), np.isnan(L[r0:r0 + Lh.size]))
        assert np.allclose(Lh, L[r0:r0 + Lh.size], rtol=1e-12, atol=1e-14, equal_nan=True)
        assert np.allclose(hh, heat[h], rtol=1e-12, atol=1e-15)
