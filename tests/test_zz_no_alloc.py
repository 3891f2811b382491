"""veda_score_tiles_noalloc (the predictor with the library's static scratch,
for callers that cannot allocate) through the C ABI: bitwise the scores of
veda_score_tiles with a caller workspace, on two calls in a row (the long
clip, whose scratch need is close to the static array's size, then the tiny
workload, smaller and with head dim 64); a plan that needs more scratch than
the array holds is refused on the host before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import veda_workloads as wl

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gpu_path as gp  # noqa: E402
from block_sparse_attention_10_amd import binding as vb  # noqa: E402
from oracle import veda_oracle as vo  # noqa: E402

STATIC_SCRATCH_BYTES = 128 << 20


def _scores_both_ways(w):
    inp = wl.make_inputs(w)
    plan = vb.Plan.from_workload(w)
    assert plan.info["score_workspace_bytes"] <= STATIC_SCRATCH_BYTES
    dev = "cuda"
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    wq, wk = inp["w_q"].to(dev), inp["w_k"].to(dev)
    qp, kp = plan.empty_perm(), plan.empty_perm()
    plan.permute(q, qp, vb.VEDA_PERMUTE_FORWARD)
    plan.permute(k, kp, vb.VEDA_PERMUTE_FORWARD)
    ref = torch.full((plan.info["total_pairs"],), float("nan"), dtype=torch.float32, device=dev)
    plan.score(qp, kp, wq, wk, ref, plan.empty_workspace())
    got = torch.full_like(ref, float("nan"))
    vb.veda_score_tiles_noalloc(plan.handle, qp, kp, wq, wk, got)      # the C ABI call, no workspace
    torch.cuda.synchronize()
    return inp, plan, ref, got


def test_noalloc_scores_equal_workspace_scores_two_calls():
    # first call: the long clip (26,064 tiles, 107 MB of scratch)
    w4 = wl.workload(4)
    _, plan4, ref4, got4 = _scores_both_ways(w4)
    assert plan4.info["score_workspace_bytes"] > STATIC_SCRATCH_BYTES // 2
    assert torch.equal(ref4.view(torch.int32), got4.view(torch.int32))
    # second call, smaller input (8 tiles per head, head dim 64): bitwise the
    # workspace call's scores and the oracle's
    w1 = wl.workload(1)
    inp1, plan1, ref1, got1 = _scores_both_ways(w1)
    assert torch.equal(ref1.view(torch.int32), got1.view(torch.int32))
    op = vo.Plan.from_workload(w1)
    _, _, scores = gp.oracle_front(op, inp1)
    flat = np.concatenate([s.reshape(-1) for s in scores])
    assert np.array_equal(got1.cpu().numpy().view(np.uint32), flat.view(np.uint32))


def test_noalloc_refuses_a_plan_larger_than_the_static_scratch():
    w = wl.workload(4)
    heads = 32          # 16 heads of each tile shape: 34,752 tiles > 32,768
    shapes = [w.tile_shapes[0]] * 16 + [w.tile_shapes[12]] * 16
    plan = vb.Plan(w.segments, heads, w.head_dim, shapes, w.budget_mode, w.keep_num, w.keep_den)
    assert plan.info["score_workspace_bytes"] > STATIC_SCRATCH_BYTES
    buf = torch.zeros(1 << 12, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    status = vb.lib().veda_score_tiles_noalloc(plan.handle, p, p, p, p, p, None)
    assert status == 4                      # VEDA_ERR_WORKSPACE, nothing launched
    assert "static scratch" in vb.veda_last_error()
    torch.cuda.synchronize()
