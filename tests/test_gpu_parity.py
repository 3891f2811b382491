"""GPU parity of every call of the Veda path against the CPU oracle, through
the C ABI (ctypes binding), on seeded synthetic inputs.

Bars: bit-exact for permuted tensors, scores, CSR masks and dense masks;
bf16 attention outputs within max-abs 2e-2 and relative L2 1e-2 of the fp64
oracle over valid rows; LSE within 1e-3; block heat within 1e-4.
"""

import numpy as np
import pytest
import torch

import veda_workloads as wl
from oracle import veda_oracle as vo

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import gpu_path as gp  # noqa: E402
from block_sparse_attention_10_amd import binding as vb  # noqa: E402


def setup_module(_):
    ok, why = vb.veda_available(0)
    assert ok, "libveda refuses this device: " + why


def small_workloads():
    V, DN = wl.VIDEO3D, wl.DENSE1D
    return [
        wl.Workload(90, "small_partial_d64", (wl.Segment(V, (4, 10, 12), 0),), 2, 64, ((2, 8, 8),) * 2,
                    wl.KEEP_RATIO, 1, 4),
        wl.Workload(91, "small_packed_2shapes", (wl.Segment(V, (2, 8, 12), 0), wl.Segment(V, (4, 10, 12), 192),
                                                 wl.Segment(DN, (1, 1, 200), 672)),
                    4, 128, ((2, 8, 8), (4, 4, 8), (2, 8, 8), (4, 4, 8)), wl.KEEP_RATIO, 1, 3),
        wl.Workload(92, "odd_fixed_k", (wl.Segment(V, (3, 9, 17), 0),), 3, 128,
                    ((1, 8, 16), (2, 4, 16), (1, 8, 16)), wl.FIXED_K, fixed_k=4),
        wl.Workload(93, "single_partial_tile", (wl.Segment(V, (1, 5, 7), 0),), 2, 64, ((1, 8, 16),) * 2,
                    wl.KEEP_RATIO, 1, 10),
        wl.Workload(94, "dense_only_audio", (wl.Segment(DN, (1, 1, 300), 0),), 1, 128, ((2, 8, 8),),
                    wl.KEEP_RATIO, 1, 10),
        # degenerate budgets: only the diagonal (FIXED_K 0, two tile shapes); keep ratio 0 with a
        # dense audio segment (video rows keep the diagonal and the audio tiles); keep ratio 1
        wl.Workload(87, "diag_only_fixed_k0", (wl.Segment(V, (2, 16, 24), 0),), 2, 128, ((2, 8, 8), (1, 8, 16)),
                    wl.FIXED_K, fixed_k=0),
        wl.Workload(86, "keep_zero_with_audio", (wl.Segment(V, (2, 8, 24), 0), wl.Segment(DN, (1, 1, 150), 384)),
                    2, 64, ((2, 8, 8),) * 2, wl.KEEP_RATIO, 0, 10),
        wl.Workload(88, "keep_all_ratio", (wl.Segment(V, (2, 8, 24), 0), wl.Segment(DN, (1, 1, 150), 384)),
                    2, 64, ((2, 8, 8),) * 2, wl.KEEP_RATIO, 1, 1),
    ]


def check_front(w, inp, g, rows=None):
    """Permutation, scores, CSR and dense mask: bit-exact."""
    op = vo.Plan.from_workload(w)
    qp, kp, scores = gp.oracle_front(op, inp)
    # permuted Q / K bit-exact, V in the tile-transposed layout bit-exact
    assert np.array_equal(gp.i16(g["q_perm"]), vo.permute_forward(op, gp.i16(inp["q"])))
    assert np.array_equal(gp.i16(g["k_perm"]), vo.permute_forward(op, gp.i16(inp["k"])))
    vperm = vo.permute_forward(op, gp.i16(inp["v"]))
    vt_ref = vperm.reshape(op.total_tiles, 128, w.head_dim).transpose(0, 2, 1)
    assert np.array_equal(gp.i16(g["v_t"]), vt_ref)
    # scores bit-exact
    sg = gp.split_scores(None, op, g["scores"].cpu().numpy())
    for h in range(w.num_heads):
        assert np.array_equal(sg[h].view(np.uint32), scores[h].view(np.uint32)), "scores head %d" % h
    # selection from the oracle's own scores
    sel = vo.select_blocks(op, scores)
    rp, ci = vo.to_csr(op, sel)
    assert np.array_equal(g["row_ptr"].cpu().numpy(), rp)
    assert np.array_equal(g["col_idx"].cpu().numpy(), ci)
    dm = np.concatenate([m.reshape(-1) for m in vo.to_dense_mask(op, sel)])
    assert np.array_equal(g["dense_mask"].cpu().numpy(), dm)
    return op, qp, kp, sel


def check_attention(w, inp, g, op, qp, kp, sel, rows=None):
    """O (in natural order, or permuted rows when the path produced them) and
    LSE against the oracle over valid rows; visited blocks == nnz."""
    vp = vo.permute_forward(op, gp.f64(inp["v"]))
    O, L = vo.block_sparse_attention(op, qp, kp, vp, sel, w.softmax_scale, rows=rows)
    vr = gp.valid_rows(op)
    vr = vr[~np.isnan(L[vr])]
    if g["o"] is not None:
        o_gpu = gp.f64(g["o"])
    else:   # natural-order output: bring it to permuted rows with the oracle's permutation
        o_gpu = vo.permute_forward(op, gp.f64(g["o_nat"]))
    max_abs, rel = gp.attn_errors(o_gpu, O, vr)
    lse_err = float(np.max(np.abs(g["lse"].cpu().numpy().astype(np.float64)[vr] - L[vr])))
    print("%s: rows=%d max_abs=%.3e rel_l2=%.3e lse=%.3e" % (w.name, len(vr), max_abs, rel, lse_err), flush=True)
    assert max_abs <= gp.MAX_ABS and rel <= gp.REL_L2 and lse_err <= gp.LSE_ABS
    assert int(g["visited"].item()) == op_nnz(op, sel)
    if rows is None:
        on = vo.permute_inverse(op, np.nan_to_num(O))
        got = gp.f64(g["o_nat"])
        assert np.max(np.abs(got - on)) <= gp.MAX_ABS


def op_nnz(op, sel):
    return sum(len(r) for rows in sel for r in rows)


@pytest.mark.parametrize("mode", ["fused", "separate", "layer"])
@pytest.mark.parametrize("w", small_workloads(), ids=lambda w: w.name)
def test_small_workloads(w, mode):
    """The whole path against the oracle: fused permutation and pooling,
    separate calls, and the benchmark's layer calls (no permuted Q copy, the
    attention reading Q in its natural layout)."""
    inp = wl.make_inputs(w, seed=w.index)
    g = gp.gpu_path(w, inp, fused=mode != "separate", layer=mode == "layer")
    op, qp, kp, sel = check_front(w, inp, g)
    check_attention(w, inp, g, op, qp, kp, sel)


def _guard_workload():
    # every key tile in every row (ascending), partial tiles, D = 64
    return wl.Workload(96, "guard_all_blocks", (wl.Segment(wl.VIDEO3D, (4, 10, 12), 0),), 2, 64, ((2, 8, 8),) * 2,
                       wl.ALL_BLOCKS)


def test_guard_large_late_logits():
    """Rows whose later key tiles hold logits far above their first key
    group's maximum (more than 64 log2 units): the fast pass cannot keep p
    bounded there and the kernel must fall back to exact re-basing.  Without
    the fallback those rows overflow."""
    w = _guard_workload()
    inp = wl.make_inputs(w, seed=w.index)
    op = vo.Plan.from_workload(w)
    k = inp["k"].float()
    for h in range(w.num_heads):            # scale the keys of each head's last tile by 64 (exact)
        perm = op.heads[h].perm()
        last = perm[(op.heads[h].num_tiles - 1) * 128:]
        toks = torch.from_numpy(last[last >= 0].astype(np.int64))
        k[toks, h, :] *= 64.0
    inp["k"] = k.to(torch.bfloat16)
    g = gp.gpu_path(w, inp)
    op, qp, kp, sel = check_front(w, inp, g)
    # precondition: some valid row's logits exceed its first group's maximum by > 70 (log2 units)
    c = w.softmax_scale / np.log(2.0)
    worst = 0.0
    for h in range(w.num_heads):
        o = op.row_offset[h]
        for i, row in enumerate(sel[h]):
            j0 = min(row)
            q = qp[o + 128 * i: o + 128 * (i + 1)]
            first = kp[o + 128 * j0: o + 128 * j0 + 32]
            allk = np.concatenate([kp[o + 128 * j: o + 128 * (j + 1)] for j in row])
            worst = max(worst, float(np.max((q @ allk.T).max(1) - (q @ first.T).max(1))) * c)
    assert worst > 70.0, worst
    check_attention(w, inp, g, op, qp, kp, sel)


def test_rows_longer_than_the_staged_list():
    """Rows of more than 2048 key blocks (a dense 1-D segment of 2051 tiles,
    the last one partial; one head, D = 64): the attention kernel stages a
    row's block list in LDS 2048 entries at a time and refills it mid-row.
    The plain inputs run the fast pass; with the keys of tile 2049 (past the
    refill point) scaled by 64 every row exceeds the fast pass's bound and
    the exact fallback pass, with its own refill, runs instead.  Sampled
    query tiles against the oracle over all 2051 key tiles."""
    n_tok = 128 * 2050 + 37
    w = wl.Workload(97, "long_rows_2051_tiles", (wl.Segment(wl.DENSE1D, (1, 1, n_tok), 0),), 1, 64,
                    ((2, 8, 8),), wl.KEEP_RATIO, 1, 10)
    base = wl.make_inputs(w, seed=w.index)
    op = vo.Plan.from_workload(w)
    n = op.heads[0].num_tiles
    assert n == 2051
    perm = op.heads[0].perm()
    for scaled in (False, True):
        inp = dict(base)
        if scaled:
            k = base["k"].float()
            toks = perm[128 * 2049: 128 * 2050]
            k[torch.from_numpy(toks[toks >= 0].astype(np.int64)), 0, :] *= 64.0   # exact in bf16
            inp["k"] = k.to(torch.bfloat16)
        g = gp.gpu_path(w, inp, dense_mask=False)
        rp, col = g["row_ptr"].cpu().numpy(), g["col_idx"].cpu().numpy()
        for i in range(n):      # a dense segment keeps every key tile, ascending
            assert np.array_equal(col[rp[i]:rp[i + 1]], np.arange(n))
        assert int(g["visited"].item()) == n * n
        qp, kp, vp = (vo.permute_forward(op, gp.f64(inp[x])) for x in ("q", "k", "v"))
        if scaled:   # precondition: tile 2049's logits exceed the first key group's maximum by > 70 (log2 units)
            c = w.softmax_scale / np.log(2.0)
            q0 = qp[:128]
            excess = (q0 @ kp[128 * 2049: 128 * 2050].T).max(1) - (q0 @ kp[:32].T).max(1)
            assert float(np.max(excess)) * c > 70.0
        o_nat, lse = gp.f64(g["o_nat"]), g["lse"].cpu().numpy().astype(np.float64)
        for i in (0, 1024, n - 1):
            O, L = vo.attention_row_tile(op, 0, i, qp, kp, vp, range(n), w.softmax_scale)
            nv = op.heads[0].tiles[i].valid
            got = o_nat[perm[128 * i: 128 * i + nv], 0]
            max_abs = float(np.max(np.abs(got - O)))
            rel = float(np.linalg.norm(got - O) / np.linalg.norm(O))
            lerr = float(np.max(np.abs(lse[128 * i: 128 * i + nv] - L)))
            print("long rows scaled=%s tile %d: max_abs %.3e rel_l2 %.3e lse %.3e" % (scaled, i, max_abs, rel, lerr),
                  flush=True)
            assert max_abs <= gp.MAX_ABS and rel <= gp.REL_L2 and lerr <= gp.LSE_ABS


def test_dense_lse_heat_rows_longer_than_the_staged_list():
    """The one-pass dense LSE and heat on rows of 2051 key blocks (a dense
    1-D segment, one head, D = 64; the staged block list refills mid-row and
    the heat reduction reads the rest of the row's list from memory), on the
    fast pass and, with tile 2049's keys scaled by 64, on the exact fallback
    pass with its re-walk: sampled query tiles' LSE and heat rows against the
    oracle, every heat row summing to 1."""
    n_tok = 128 * 2050 + 37
    w = wl.Workload(97, "long_rows_2051_tiles", (wl.Segment(wl.DENSE1D, (1, 1, n_tok), 0),), 1, 64,
                    ((2, 8, 8),), wl.ALL_BLOCKS)
    base = wl.make_inputs(w, seed=w.index)
    op = vo.Plan.from_workload(w)
    n = op.heads[0].num_tiles
    perm = op.heads[0].perm()
    for scaled in (False, True):
        inp = dict(base)
        if scaled:
            k = base["k"].float()
            toks = perm[128 * 2049: 128 * 2050]
            k[torch.from_numpy(toks[toks >= 0].astype(np.int64)), 0, :] *= 64.0
            inp["k"] = k.to(torch.bfloat16)
        g = gp.gpu_path(w, inp, dense_mask=False)
        lse, heat = _dense_lse_heat(g, w)
        a, b = g["lse"].cpu().numpy(), lse.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        hg = heat.cpu().numpy().reshape(n, n)
        assert np.max(np.abs(hg.sum(axis=1) - 1.0)) <= 1e-3
        qp, kp, vp = (vo.permute_forward(op, gp.f64(inp[x])) for x in ("q", "k", "v"))
        sampled = (0, 1024, n - 1)
        L = np.full(op.total_rows, np.nan)
        for i in sampled:
            _, Li = vo.attention_row_tile(op, 0, i, qp, kp, vp, range(n), w.softmax_scale)
            nv = op.heads[0].tiles[i].valid
            L[128 * i: 128 * i + nv] = Li
            assert np.max(np.abs(b[128 * i: 128 * i + nv] - Li)) <= gp.LSE_ABS
        ref = vo.block_heat(op, qp, kp, L, w.softmax_scale, rows=sampled)[0]
        for i in sampled:
            err = float(np.max(np.abs(hg[i] - ref[i])))
            print("long rows scaled=%s tile %d: heat max_abs %.3e" % (scaled, i, err), flush=True)
            assert err <= gp.HEAT_ABS


@pytest.mark.parametrize("kind", ["small", "guard_all_blocks", "guard_late_logits"])
def test_lse_only_equals_full_attention(kind):
    """veda_block_sparse_attn_fwd with o = NULL computes only the LSE (no PV
    products): bitwise equal to the LSE of the full call, on the fast pass
    and on the fallback pass (forced by late logits)."""
    ws = small_workloads() if kind == "small" else [_guard_workload()]
    for w in ws:
        inp = wl.make_inputs(w, seed=w.index)
        if kind == "guard_late_logits":
            op = vo.Plan.from_workload(w)
            k = inp["k"].float()
            for h in range(w.num_heads):
                perm = op.heads[h].perm()
                last = perm[(op.heads[h].num_tiles - 1) * 128:]
                k[torch.from_numpy(last[last >= 0].astype(np.int64)), h, :] *= 64.0
            inp["k"] = k.to(torch.bfloat16)
        g = gp.gpu_path(w, inp, dense_mask=False)
        plan = g["plan"]
        lse2 = torch.full_like(g["lse"], float("nan"))
        visited = torch.zeros(1, dtype=torch.int32, device="cuda")
        plan.attention(g["q_perm"], g["k_perm"], g["v_t"], g["row_ptr"], g["col_idx"], w.softmax_scale, None, lse2,
                       visited)
        torch.cuda.synchronize()
        a, b = g["lse"].cpu().numpy(), lse2.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), w.name
        assert int(visited.item()) == int(g["visited"].item())


def test_guard_padding_mass():
    """Rows whose valid logits all sit far below zero while their key tiles
    have padding slots (logit exactly 0): the padding mass the fast pass
    removes dwarfs the valid sum, so the kernel must fall back to explicit
    masking."""
    w = _guard_workload()
    inp = wl.make_inputs(w, seed=w.index)
    gen = torch.Generator().manual_seed(7)
    q = 0.1 * torch.randn(inp["q"].shape, generator=gen)
    k = 0.1 * torch.randn(inp["k"].shape, generator=gen)
    q[..., 0] += 20.0
    k[..., 0] -= 20.0                       # every logit about -400 * scale
    inp["q"], inp["k"] = q.to(torch.bfloat16), k.to(torch.bfloat16)
    g = gp.gpu_path(w, inp)
    op, qp, kp, sel = check_front(w, inp, g)
    padded = [j for h in range(w.num_heads) for row in sel[h] for j in row if op.heads[h].valid_counts()[j] < 128]
    assert padded, "the workload must select partial key tiles"
    check_attention(w, inp, g, op, qp, kp, sel)


def test_heat_masked_variant():
    """Block heat where exp(-lse) is large (all logits far below zero, partial
    tiles): the heat kernel must mask padding keys explicitly rather than
    subtract their terms."""
    w = _guard_workload()
    inp = wl.make_inputs(w, seed=w.index)
    gen = torch.Generator().manual_seed(9)
    q = 0.1 * torch.randn(inp["q"].shape, generator=gen)
    k = 0.1 * torch.randn(inp["k"].shape, generator=gen)
    q[..., 0] += 20.0
    k[..., 0] -= 20.0
    inp["q"], inp["k"] = q.to(torch.bfloat16), k.to(torch.bfloat16)
    g = gp.gpu_path(w, inp)                  # ALL budget: its LSE is the dense LSE
    plan = g["plan"]
    heat = torch.empty(plan.info["total_pairs"], dtype=torch.float32, device="cuda")
    plan.heat(g["q_perm"], g["k_perm"], g["lse"], w.softmax_scale, heat)
    torch.cuda.synchronize()
    op = vo.Plan.from_workload(w)
    qp, kp, _ = gp.oracle_front(op, inp)
    _, L = vo.block_sparse_attention(op, qp, kp, kp, vo.all_blocks_selection(op), w.softmax_scale)
    assert np.nanmax(L) < -20.0                # exp(-lse) far above 1/16
    heat_ref = vo.block_heat(op, qp, kp, L, w.softmax_scale)
    heat_gpu = gp.split_scores(None, op, heat.cpu().numpy())
    for h in range(w.num_heads):
        assert np.max(np.abs(heat_gpu[h] - heat_ref[h])) <= gp.HEAT_ABS, h


def _search_case(kind):
    """(segments, heads, dim, candidates, budget (mode, num, den, k), host samples)."""
    cands = ((1, 8, 16), (2, 8, 8), (4, 4, 8))
    if kind == "frame_local":
        segs = (wl.Segment(wl.VIDEO3D, (4, 8, 16), 0),)
        N, H, D = 512, 2, 64
        t_of = np.arange(N) // 128
        samples = []
        for s in range(2):
            g = np.random.default_rng(100 + s)
            base = np.zeros((N, H, D))
            base[np.arange(N), :, t_of] = 10.0
            samples.append(tuple(torch.from_numpy(base * m + 0.05 * g.standard_normal((N, H, D))).to(torch.bfloat16)
                                 for m in (1.0, 1.0, 0.0)))
        return segs, H, D, cands, (wl.FIXED_K, 1, 10, 2), samples
    # locality-biased layer: fixed per-head length scales, new noise per sample
    w = wl.Workload(97, "search_layer", (wl.Segment(wl.VIDEO3D, (4, 16, 16), 0),), 4, 64, ((2, 8, 8),) * 4,
                    wl.KEEP_RATIO, 1, 4)
    samples = []
    for s in range(2):
        x = wl.make_inputs(w, seed=500 + s, bias_seed=97)
        samples.append((x["q"], x["k"], x["v"]))
    return w.segments, 4, 64, cands, (wl.KEEP_RATIO, 1, 4, 0), samples


@pytest.mark.parametrize("kind", ["frame_local", "biased_layer"])
def test_tile_plan_search(kind):
    """Error table of the GPU search against the oracle's (tolerance from the
    bf16 rounding of the two outputs compared), the vote bit-exact against
    the oracle's vote on the same GPU table, and the chosen shapes against
    the oracle's own choice where its margins are clear."""
    from block_sparse_attention_10_amd import search
    segs, H, D, cands, (mode, num, den, fk), samples = _search_case(kind)
    scale = 1.0 / np.sqrt(D)
    dev_samples = [tuple(t.to("cuda") for t in smp) for smp in samples]
    err, choice = search.tile_plan_search(segs, H, D, cands, mode, num, den, fk, dev_samples, scale)
    ref = vo.tile_plan_errors(segs, H, D, cands, mode, num, den, fk,
                              [tuple(gp.f64(t) for t in smp) for smp in samples], scale)
    print("%s: gpu err %s oracle err %s" % (kind, np.round(err, 5).tolist(), np.round(ref, 5).tolist()), flush=True)
    tol = 2.0 * np.sqrt(ref) * 2.0 ** -7 + 2.0 ** -13
    assert np.all(np.abs(err - ref) <= tol), np.abs(err - ref) - tol
    assert np.array_equal(choice, vo.vote_tile_shapes(err, 2))
    ref_choice = vo.vote_tile_shapes(ref, 2)
    for h in range(H):   # where no sample's best candidate is within the tolerance of another
        clear = all(np.sort(ref[s, :, h])[1] - np.sort(ref[s, :, h])[0] > 2 * tol[s].max() for s in range(len(samples)))
        if clear:
            assert choice[h] == ref_choice[h], h


def _backward_case(w, seed, oracle=True):
    """GPU forward (permuted O and LSE), transposed lists and backward for a
    random upstream gradient; returns the GPU tensors and the oracle's fp64
    gradients on the same inputs."""
    inp = wl.make_inputs(w, seed=seed)
    g = gp.gpu_path(w, inp)
    plan, dev = g["plan"], "cuda"
    gen = torch.Generator().manual_seed(seed + 1)
    do_nat = torch.randn((w.num_tokens, w.num_heads, w.head_dim), generator=gen).to(torch.bfloat16)
    vp, dop, o = plan.empty_perm(), plan.empty_perm(), plan.empty_perm()
    plan.permute(inp["v"].to(dev), vp, vb.VEDA_PERMUTE_FORWARD)
    plan.permute(do_nat.to(dev), dop, vb.VEDA_PERMUTE_FORWARD)
    lse = torch.empty(plan.R, dtype=torch.float32, device=dev)
    plan.attention(g["q_perm"], g["k_perm"], g["v_t"], g["row_ptr"], g["col_idx"], w.softmax_scale, o, lse)
    col_ptr = torch.empty(plan.T + 1, dtype=torch.int32, device=dev)
    row_idx = torch.empty(plan.info["nnz"], dtype=torch.int32, device=dev)
    plan.transpose(g["row_ptr"], g["col_idx"], col_ptr, row_idx, plan.empty_bytes("transpose_workspace_bytes"))
    dq, dk, dv = plan.empty_perm(), plan.empty_perm(), plan.empty_perm()
    # every byte of the workspace starts as 0xff (NaN as bf16 or fp32): a dS
    # block the dQ pass read before the dK/dV pass wrote it would show up
    ws = plan.empty_bytes("bwd_workspace_bytes").fill_(255)
    plan.backward(g["q_perm"], g["k_perm"], vp, o, dop, lse, g["row_ptr"], g["col_idx"], col_ptr, row_idx,
                  w.softmax_scale, dq, dk, dv, ws)
    torch.cuda.synchronize()
    op = vo.Plan.from_workload(w)
    sel = _csr_to_selection(op, g["row_ptr"].cpu().numpy(), g["col_idx"].cpu().numpy())
    if not oracle:
        return op, sel, col_ptr, row_idx, {"inputs": (g["q_perm"], g["k_perm"], vp, dop), "grads": (dq, dk, dv),
                                           "plan": plan, "o": o, "lse": lse, "row_ptr": g["row_ptr"],
                                           "col_idx": g["col_idx"]}, None
    ref = vo.block_sparse_attention_backward(op, gp.f64(g["q_perm"]), gp.f64(g["k_perm"]), gp.f64(vp), gp.f64(dop),
                                             sel, w.softmax_scale)
    return op, sel, col_ptr, row_idx, (dq, dk, dv), ref


@pytest.mark.parametrize("w", [small_workloads()[0], small_workloads()[1], small_workloads()[3], wl.workload(2)],
                         ids=lambda w: w.name)
def test_backward(w):
    """Transposed lists bit-exact; dQ, dK, dV against the fp64 oracle over
    valid rows (bars derived like the forward's: bf16 P and dS, bf16 outputs),
    padding rows exactly zero."""
    op, sel, col_ptr, row_idx, got, ref = _backward_case(w, w.index)
    tr = vo.mask_transpose(op, sel)
    counts = [len(c) for rows in tr for c in rows]
    cp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ri = np.concatenate([c for rows in tr for c in rows]).astype(np.int32)
    assert np.array_equal(col_ptr.cpu().numpy(), cp) and np.array_equal(row_idx.cpu().numpy(), ri)
    vr = gp.valid_rows(op)
    pad = np.setdiff1d(np.arange(op.total_rows), vr)
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        a = gp.f64(a)
        d = a[vr] - b[vr]
        max_abs = float(np.max(np.abs(d)))
        rel = float(np.linalg.norm(d) / np.linalg.norm(b[vr]))
        print("%s %s: max_abs %.3e (ref max %.3e) rel_l2 %.3e" % (w.name, name, max_abs, np.max(np.abs(b[vr])), rel),
              flush=True)
        assert rel <= gp.REL_L2 and max_abs <= gp.MAX_ABS * max(1.0, float(np.max(np.abs(b[vr]))))
        assert not np.any(a[pad]), name


def test_oracle_mask_mass_and_recall():
    """Oracle mask (veda_select_blocks on the block heat) and the attention
    mass of the predicted and oracle masks (veda_mask_mass) against the
    oracle: CSR bit-exact from the same fp32 heat, masses to fp64 rounding;
    recall <= 1 (the oracle mask is the best mask under the same budgets)."""
    w = small_workloads()[1]                  # two video segments + audio, two tile shapes, D = 128
    inp = wl.make_inputs(w, seed=w.index)
    g = gp.gpu_path(w, inp)
    plan, dev = g["plan"], "cuda"
    dense = vb.Plan.from_workload(w, budget_mode=wl.ALL_BLOCKS)
    d_rp = torch.empty(plan.T + 1, dtype=torch.int32, device=dev)
    d_col = torch.empty(dense.info["nnz"], dtype=torch.int32, device=dev)
    dense.select(g["scores"], d_rp, d_col)
    d_o, d_lse = dense.empty_perm(), torch.empty(plan.R, dtype=torch.float32, device=dev)
    dense.attention(g["q_perm"], g["k_perm"], g["v_t"], d_rp, d_col, w.softmax_scale, d_o, d_lse)
    heat = torch.empty(plan.info["total_pairs"], dtype=torch.float32, device=dev)
    plan.heat(g["q_perm"], g["k_perm"], d_lse, w.softmax_scale, heat)
    o_rp = torch.empty(plan.T + 1, dtype=torch.int32, device=dev)
    o_col = torch.empty(plan.info["nnz"], dtype=torch.int32, device=dev)
    plan.select(heat, o_rp, o_col)
    m_pred = torch.empty(w.num_heads, dtype=torch.float64, device=dev)
    m_orc = torch.empty(w.num_heads, dtype=torch.float64, device=dev)
    plan.mask_mass(heat, g["row_ptr"], g["col_idx"], m_pred)
    plan.mask_mass(heat, o_rp, o_col, m_orc)
    torch.cuda.synchronize()

    op = vo.Plan.from_workload(w)
    heat_gpu = gp.split_scores(None, op, heat.cpu().numpy())
    sel_o = vo.oracle_mask(op, heat_gpu)
    rp, ci = vo.to_csr(op, sel_o)
    assert np.array_equal(o_rp.cpu().numpy(), rp) and np.array_equal(o_col.cpu().numpy(), ci)
    sel_p = _csr_to_selection(op, g["row_ptr"].cpu().numpy(), g["col_idx"].cpu().numpy())
    ref_p, ref_o = vo.mask_mass(op, heat_gpu, sel_p), vo.mask_mass(op, heat_gpu, sel_o)
    got_p, got_o = m_pred.cpu().numpy(), m_orc.cpu().numpy()
    assert np.max(np.abs(got_p - ref_p) / ref_p) < 1e-12 and np.max(np.abs(got_o - ref_o) / ref_o) < 1e-12
    r = got_p / got_o
    print("oracle mask mass %s recall %s" % (np.round(got_o, 4), np.round(r, 4)), flush=True)
    assert np.all(r <= 1.0 + 1e-12) and np.all(got_o <= 1.0 + 1e-6) and np.all(got_p > 0.0)
    # the GPU heat itself against the oracle's (dense LSE in fp64)
    qp, kp, _ = gp.oracle_front(op, inp)
    _, L = vo.block_sparse_attention(op, qp, kp, kp, vo.all_blocks_selection(op), w.softmax_scale)
    heat_ref = vo.block_heat(op, qp, kp, L, w.softmax_scale)
    for h in range(w.num_heads):
        assert np.max(np.abs(heat_gpu[h] - heat_ref[h])) <= gp.HEAT_ABS


def test_backward_deterministic_and_workspace_independent():
    """The backward twice on the same inputs, the second time over a
    workspace cleared to zero instead of 0xff: dQ, dK, dV bitwise equal (dS
    goes through the workspace, but every block is written before it is
    read, and all sums run in a fixed order)."""
    w = small_workloads()[1]
    op, sel, col_ptr, row_idx, got, _ = _backward_case(w, w.index, oracle=False)
    g = got["grads"]
    q, k, vp, dop = got["inputs"]
    plan = got["plan"]
    dq2, dk2, dv2 = plan.empty_perm(), plan.empty_perm(), plan.empty_perm()
    ws = plan.empty_bytes("bwd_workspace_bytes").zero_()
    plan.backward(q, k, vp, got["o"], dop, got["lse"], got["row_ptr"], got["col_idx"], col_ptr, row_idx,
                  w.softmax_scale, dq2, dk2, dv2, ws)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), g, (dq2, dk2, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        assert torch.isfinite(a.float()).all(), name


def test_backward_config3_one_head():
    """The bench's backward configuration (the 16x30x54 clip, 24 heads, full
    size): transposed lists bit-exact on every head; dQ, dK, dV of one whole
    head (all its rows, so every key tile's full column) against the fp64
    oracle run on that head alone, from the same permuted inputs and mask."""
    w = wl.workload(3)
    op, sel, col_ptr, row_idx, got, _ = _backward_case(w, w.index, oracle=False)
    tr = vo.mask_transpose(op, sel)
    counts = [len(c) for rows in tr for c in rows]
    cp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ri = np.concatenate([c for rows in tr for c in rows]).astype(np.int32)
    assert np.array_equal(col_ptr.cpu().numpy(), cp) and np.array_equal(row_idx.cpu().numpy(), ri)
    h = 7
    sub = vo.Plan(w.segments, 1, w.head_dim, [w.tile_shapes[h]], w.budget_mode, w.keep_num, w.keep_den, w.fixed_k)
    r0, L = op.row_offset[h], sub.total_rows
    q, k, v, do = (gp.f64(t)[r0:r0 + L] for t in got["inputs"])
    ref = vo.block_sparse_attention_backward(sub, q, k, v, do, [sel[h]], w.softmax_scale)
    vr = gp.valid_rows(sub)
    for name, a, b in zip(("dq", "dk", "dv"), got["grads"], ref):
        a = gp.f64(a)[r0:r0 + L]
        d = a[vr] - b[vr]
        max_abs = float(np.max(np.abs(d)))
        rel = float(np.linalg.norm(d) / np.linalg.norm(b[vr]))
        print("config 3 head %d %s: max_abs %.3e (ref max %.3e) rel_l2 %.3e" % (h, name, max_abs,
              np.max(np.abs(b[vr])), rel), flush=True)
        assert rel <= gp.REL_L2 and max_abs <= gp.MAX_ABS * max(1.0, float(np.max(np.abs(b[vr]))))
        assert not np.any(a[np.setdiff1d(np.arange(L), vr)]), name


def _csr_to_selection(op, row_ptr, col):
    sel, t = [], 0
    for h in range(op.num_heads):
        rows = []
        for _ in range(op.heads[h].num_tiles):
            rows.append(col[row_ptr[t]:row_ptr[t + 1]].astype(np.int64))
            t += 1
        sel.append(rows)
    return sel


@pytest.mark.parametrize("idx", [1, 2, 3])
def test_config_full(idx):
    w = wl.workload(idx)
    inp = wl.make_inputs(w)
    g = gp.gpu_path(w, inp)
    op, qp, kp, sel = check_front(w, inp, g)
    check_attention(w, inp, g, op, qp, kp, sel)


def test_config2_separate_calls():
    w = wl.workload(2)
    inp = wl.make_inputs(w)
    g = gp.gpu_path(w, inp, fused=False)
    op, qp, kp, sel = check_front(w, inp, g)
    check_attention(w, inp, g, op, qp, kp, sel)


def _order_sensitive_inputs(w):
    """Inputs whose projections depend on the order of the fp64 sum: channel
    5 of Q and channel 9 of K are constant (so a tile's mean, max and min of
    that channel are equal), and W gives the mean column +2^40 and the min
    column -2^40 of that channel.  Summed in ascending e, the big term enters
    at e = c, every term up to e = 2D + c is rounded against it (ulp 2^-12),
    and it cancels exactly at e = 2D + c; another order rounds differently."""
    inp = wl.make_inputs(w)
    D = w.head_dim
    inp["q"][:, :, 5] = 0.75
    inp["k"][:, :, 9] = -1.25
    for key, c in (("w_q", 5), ("w_k", 9)):
        wt = inp[key].clone()
        wt[:, :, c] = 2.0 ** 40
        wt[:, :, 2 * D + c] = -(2.0 ** 40)
        inp[key] = wt
    return inp


def _project_blocked(op, feats, w):
    """The projection with each step's four products summed first (the
    alternative order a matrix instruction could take), for the check that
    the inputs above tell the orders apart."""
    H, D, E = w.shape
    out = np.zeros((op.total_tiles, D), dtype=np.float32)
    for h in range(H):
        t0, t1 = op.tile_offset[h], op.tile_offset[h + 1]
        f = feats[t0:t1].astype(np.float64)
        wh = w[h].astype(np.float64)
        acc = f[:, 0:D].copy()
        for e in range(0, E, 4):
            p = [f[:, e + u:e + u + 1] * wh[:, e + u][None, :] for u in range(4)]
            acc += (p[0] + p[1]) + (p[2] + p[3])
        out[t0:t1] = acc.astype(np.float32)
    return out


def test_predictor_sums_follow_the_sequential_order():
    """Projections and scores bit-exact against the oracle's ascending-order
    fp64 sums on inputs where the summation order shows in the fp32 result."""
    w = wl.workload(2)
    inp = _order_sensitive_inputs(w)
    op = vo.Plan.from_workload(w)
    qn, kn = gp.f64(inp["q"]), gp.f64(inp["k"])
    fq = vo.pool_tiles(op, vo.permute_forward(op, qn))
    fk = vo.pool_tiles(op, vo.permute_forward(op, kn))
    qh = vo.project(op, fq, inp["w_q"].numpy())
    kh = vo.project(op, fk, inp["w_k"].numpy())
    scores = vo.score_pairs(op, qh, kh)
    # the inputs separate the orders: a blocked sum gives other fp32 values
    assert np.count_nonzero(_project_blocked(op, fq, inp["w_q"].numpy()) != qh) > qh.size // 10
    plan = vb.Plan.from_workload(w)
    dev = "cuda"
    q, k, v = (inp[x].to(dev).to(torch.bfloat16) for x in ("q", "k", "v"))
    qp, kp, vt, ws = plan.empty_perm(), plan.empty_perm(), plan.empty_vt(), plan.empty_workspace()
    sc = torch.empty(plan.info["total_pairs"], dtype=torch.float32, device=dev)
    plan.permute_qkv(q, k, v, qp, kp, vt, ws)
    plan.score_pooled(inp["w_q"].to(dev), inp["w_k"].to(dev), sc, ws)
    torch.cuda.synchronize()
    views = plan.score_workspace_views(ws)
    hq = views["q_hat"].cpu().numpy()
    hk = views["k_hat"].cpu().numpy()
    assert np.array_equal(hq.view(np.uint32), qh.view(np.uint32))
    assert np.array_equal(hk.view(np.uint32), kh.view(np.uint32))
    sg = gp.split_scores(None, op, sc.cpu().numpy())
    for h in range(w.num_heads):
        assert np.array_equal(sg[h].view(np.uint32), scores[h].view(np.uint32)), "scores head %d" % h


def test_fused_equals_separate_bitwise():
    w = wl.workload(3)
    inp = wl.make_inputs(w)
    a = gp.gpu_path(w, inp, fused=True)
    b = gp.gpu_path(w, inp, fused=False)
    for key in ("q_perm", "k_perm", "v_t", "scores", "col_idx", "lse", "o_nat"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("idx", [2, 4])
def test_permute_qk_only_and_side_stream_v(idx):
    """veda_permute_qkv with v = v_t = NULL (Q and K only, with the pooling)
    and V's tile-transposed permutation on a second stream, the way the bench
    runs a layer: bitwise equal to the three-tensor fused call (permuted Q, K,
    V^T and the pooled features); config 4 has two tile shapes."""
    w = wl.workload(idx)
    inp = wl.make_inputs(w)
    plan = vb.Plan.from_workload(w)
    dev = "cuda"
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    ref = [plan.empty_perm(), plan.empty_perm(), plan.empty_vt(), plan.empty_workspace()]
    plan.permute_qkv(q, k, v, *ref)
    got = [torch.full_like(ref[0], -1), torch.full_like(ref[1], -1), torch.full_like(ref[2], -1),
           torch.full_like(ref[3], float("nan"))]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.permute(v, got[2], vb.VEDA_PERMUTE_FORWARD_TRANSPOSED, stream=side)
    plan.permute_qkv(q, k, None, got[0], got[1], None, got[3])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    rv, gv = plan.score_workspace_views(ref[3]), plan.score_workspace_views(got[3])
    ref[3] = torch.cat([rv["feat_q"].reshape(-1), rv["feat_k"].reshape(-1)])
    got[3] = torch.cat([gv["feat_q"].reshape(-1), gv["feat_k"].reshape(-1)])
    for a, b, name in zip(ref, got, ("q_perm", "k_perm", "v_t", "pooled features")):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), name
    with pytest.raises(ValueError):
        plan.permute_qkv(q, k, v, got[0], got[1], None, got[3])
    with pytest.raises(vb.VedaError) as e:
        vb.veda_permute_qkv(plan.handle, q, k, v, got[0], got[1], None, got[3])
    assert e.value.status == 1                   # VEDA_ERR_INVALID_ARG: v without v_t


@pytest.mark.parametrize("which", ["small", "config3"])
def test_natural_q_layout(which):
    """Q in its natural [N, H, D] layout (q_layout NATURAL, gathered through
    the slot -> token table) against the permuted copy: the attention's O and
    LSE, and the dense LSE and heat, bitwise equal; veda_permute_qkv with
    q_perm = NULL writes K, V^T and the pooled features of Q and K bitwise
    as the full call does (ragged tiles, two tile shapes, D = 64 and 128,
    packed segments, the 16:9 clip)."""
    ws = small_workloads() if which == "small" else [wl.workload(3)]
    for w in ws:
        inp = wl.make_inputs(w, seed=w.index)
        g = gp.gpu_path(w, inp)
        plan, dev = g["plan"], "cuda"
        q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
        # the layer's permutation without the Q copy
        got = [torch.full_like(g["k_perm"], -1), torch.full_like(g["v_t"], -1),
               torch.full_like(plan.empty_workspace(), float("nan"))]
        ref_ws = plan.empty_workspace()
        plan.permute_qkv(q, k, v, plan.empty_perm(), plan.empty_perm(), plan.empty_vt(), ref_ws)
        plan.permute_qkv(q, k, v, None, got[0], got[1], got[2])
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), g["k_perm"].view(torch.int16)), w.name
        assert torch.equal(got[1].view(torch.int16), g["v_t"].view(torch.int16)), w.name
        rv, gv = plan.score_workspace_views(ref_ws), plan.score_workspace_views(got[2])
        for key in ("feat_q", "feat_k"):
            assert torch.equal(rv[key].view(torch.int32), gv[key].view(torch.int32)), (w.name, key)
        # attention: permuted Q against natural Q, O in both layouts
        for o_layout in (vb.VEDA_LAYOUT_NATURAL, vb.VEDA_LAYOUT_PERMUTED):
            shape = (w.num_tokens, w.num_heads, w.head_dim) if o_layout == vb.VEDA_LAYOUT_NATURAL else (plan.R, w.head_dim)
            outs = []
            for q_in, q_layout in ((g["q_perm"], vb.VEDA_LAYOUT_PERMUTED), (q, vb.VEDA_LAYOUT_NATURAL)):
                o = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
                lse = torch.full((plan.R,), float("nan"), dtype=torch.float32, device=dev)
                plan.attention(q_in, g["k_perm"], g["v_t"], g["row_ptr"], g["col_idx"], w.softmax_scale, o, lse,
                               o_layout=o_layout, q_layout=q_layout)
                outs.append((o, lse))
            torch.cuda.synchronize()
            (o0, l0), (o1, l1) = outs
            assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)), (w.name, o_layout)
            assert torch.equal(l0.view(torch.int32), l1.view(torch.int32)), (w.name, o_layout)
        # the dense LSE and heat
        if which == "small":
            gd = gp.gpu_path(w, inp, budget_mode=wl.ALL_BLOCKS, dense_mask=False)
            pd = gd["plan"]
            res = []
            for q_in, q_layout in ((gd["q_perm"], vb.VEDA_LAYOUT_PERMUTED), (q, vb.VEDA_LAYOUT_NATURAL)):
                lse = torch.full((pd.R,), float("nan"), dtype=torch.float32, device=dev)
                heat = torch.full((pd.info["total_pairs"],), float("nan"), dtype=torch.float32, device=dev)
                wsh = torch.full((pd.info["heat_workspace_bytes"] // 4,), float("nan"), dtype=torch.float32,
                                 device=dev)
                pd.lse_heat(q_in, gd["k_perm"], gd["row_ptr"], gd["col_idx"], w.softmax_scale, lse, heat, wsh,
                            q_layout=q_layout)
                res.append((lse, heat))
            torch.cuda.synchronize()
            assert torch.equal(res[0][0].view(torch.int32), res[1][0].view(torch.int32)), w.name
            assert torch.equal(res[0][1].view(torch.int32), res[1][1].view(torch.int32)), w.name


def test_all_mask_equals_dense_attention():
    """The ALL budget through the same kernels is dense attention (library fp64 SDPA)."""
    w = wl.Workload(95, "dense_small", (wl.Segment(wl.VIDEO3D, (4, 10, 12), 0),), 2, 128, ((2, 8, 8),) * 2,
                    wl.ALL_BLOCKS)
    inp = wl.make_inputs(w, seed=95)
    g = gp.gpu_path(w, inp)
    O, L = vo.dense_attention(gp.f64(inp["q"]), gp.f64(inp["k"]), gp.f64(inp["v"]), w.softmax_scale)
    got = gp.f64(g["o_nat"])
    diff = got - O
    assert np.max(np.abs(diff)) <= gp.MAX_ABS
    assert np.linalg.norm(diff) / np.linalg.norm(O) <= gp.REL_L2


def test_deterministic_bitwise():
    w = wl.workload(2)
    inp = wl.make_inputs(w)
    a = gp.gpu_path(w, inp)
    b = gp.gpu_path(w, inp)
    for key in ("scores", "col_idx", "o_nat", "lse"):
        assert torch.equal(a[key], b[key]), key


def _late_logits(w, inp):
    """Scale the keys of every head's last key tile by 64: logits there lie far
    above the first key group's maximum, which forces the exact fallback pass."""
    op = vo.Plan.from_workload(w)
    k = inp["k"].float()
    for h in range(w.num_heads):
        perm = op.heads[h].perm()
        last = perm[(op.heads[h].num_tiles - 1) * 128:]
        k[torch.from_numpy(last[last >= 0].astype(np.int64)), h, :] *= 64.0
    inp["k"] = k.to(torch.bfloat16)


def _far_below_zero(inp, seed):
    """Every logit about -400 * scale while key tiles have padding slots: the
    padding mass the fast pass removes dwarfs the valid sum (fallback pass)."""
    gen = torch.Generator().manual_seed(seed)
    q = 0.1 * torch.randn(inp["q"].shape, generator=gen)
    k = 0.1 * torch.randn(inp["k"].shape, generator=gen)
    q[..., 0] += 20.0
    k[..., 0] -= 20.0
    inp["q"], inp["k"] = q.to(torch.bfloat16), k.to(torch.bfloat16)


def _dense_lse_heat(g, w):
    plan = g["plan"]
    lse = torch.full_like(g["lse"], float("nan"))
    heat = torch.full((plan.info["total_pairs"],), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((plan.info["heat_workspace_bytes"] // 4,), float("nan"), dtype=torch.float32, device="cuda")
    plan.lse_heat(g["q_perm"], g["k_perm"], g["row_ptr"], g["col_idx"], w.softmax_scale, lse, heat, ws)
    torch.cuda.synchronize()
    return lse, heat


@pytest.mark.parametrize("kind", ["small", "guard_all_blocks", "guard_late_logits", "guard_far_below_zero"])
def test_dense_lse_heat(kind):
    """veda_dense_lse_heat (dense LSE and block heat in one pass): the LSE is
    bitwise equal to the attention's over the same all-blocks CSR; the heat
    matches the oracle's heat from its own dense LSE and veda_block_heat on
    the same LSE (HEAT_ABS), on the fast pass and on the fallback pass (late
    logits; logits far below zero with partial key tiles)."""
    ws = small_workloads() if kind == "small" else [_guard_workload()]
    for w in ws:
        inp = wl.make_inputs(w, seed=w.index)
        if kind == "guard_late_logits":
            _late_logits(w, inp)
        elif kind == "guard_far_below_zero":
            _far_below_zero(inp, 9)
        g = gp.gpu_path(w, inp, budget_mode=wl.ALL_BLOCKS, dense_mask=False)
        plan = g["plan"]
        lse, heat = _dense_lse_heat(g, w)
        a, b = g["lse"].cpu().numpy(), lse.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), w.name
        heat2 = torch.empty_like(heat)
        plan.heat(g["q_perm"], g["k_perm"], g["lse"], w.softmax_scale, heat2)
        torch.cuda.synchronize()
        op = vo.Plan.from_workload(w)
        qp, kp, _ = gp.oracle_front(op, inp)
        _, L = vo.block_sparse_attention(op, qp, kp, kp, vo.all_blocks_selection(op), w.softmax_scale)
        ref = vo.block_heat(op, qp, kp, L, w.softmax_scale)
        hg = gp.split_scores(None, op, heat.cpu().numpy())
        h2 = gp.split_scores(None, op, heat2.cpu().numpy())
        for h in range(w.num_heads):
            err = float(np.max(np.abs(hg[h] - ref[h])))
            print("%s %s head %d: heat max_abs %.3e (two-pass %.3e)" % (kind, w.name, h, err,
                  float(np.max(np.abs(h2[h] - ref[h])))), flush=True)
            assert err <= gp.HEAT_ABS, (w.name, h)
            assert np.max(np.abs(hg[h] - h2[h])) <= gp.HEAT_ABS, (w.name, h)


def test_dense_lse_heat_errors():
    """The fused call refuses a plan that is not all-blocks (UNSUPPORTED) and a
    short workspace (WORKSPACE) on the host, before any launch."""
    w = _guard_workload()
    inp = wl.make_inputs(w, seed=w.index)
    g = gp.gpu_path(w, inp, budget_mode=wl.ALL_BLOCKS, dense_mask=False)
    plan = g["plan"]
    heat = torch.empty(plan.info["total_pairs"], dtype=torch.float32, device="cuda")
    short = torch.empty(plan.info["heat_workspace_bytes"] // 4 - 64, dtype=torch.float32, device="cuda")
    with pytest.raises(vb.VedaError) as e:
        vb.veda_dense_lse_heat(plan.handle, g["q_perm"], g["k_perm"], g["row_ptr"], g["col_idx"], w.softmax_scale,
                               g["lse"], heat, short)
    assert e.value.status == 4          # VEDA_ERR_WORKSPACE
    sparse = vb.Plan.from_workload(w, budget_mode=wl.KEEP_RATIO)
    ws = torch.empty(plan.info["heat_workspace_bytes"] // 4, dtype=torch.float32, device="cuda")
    with pytest.raises(vb.VedaError) as e:
        vb.veda_dense_lse_heat(sparse.handle, g["q_perm"], g["k_perm"], g["row_ptr"], g["col_idx"],
                               w.softmax_scale, g["lse"], heat, ws)
    assert e.value.status == 3          # VEDA_ERR_UNSUPPORTED


def test_error_paths_on_device():
    w = wl.workload(1)
    plan = vb.Plan.from_workload(w)
    with pytest.raises(ValueError):
        plan.permute(torch.zeros(3, device="cuda", dtype=torch.bfloat16), plan.empty_perm(), 0)
    lib = vb.lib()
    import ctypes
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    # misaligned pointer -> INVALID_ARG before any launch
    assert lib.veda_permute_tiles(plan.handle, buf.data_ptr() + 2, buf.data_ptr() + 4096, 0, None) == 1
    assert lib.veda_block_sparse_attn_fwd(plan.handle, buf.data_ptr(), 0, buf.data_ptr(), buf.data_ptr(),
                                          buf.data_ptr(), buf.data_ptr(), ctypes.c_float(float("nan")),
                                          buf.data_ptr(), 0, None, None, None) == 1
    assert lib.veda_block_sparse_attn_fwd(plan.handle, buf.data_ptr(), 0, buf.data_ptr(), buf.data_ptr(),
                                          buf.data_ptr(), buf.data_ptr(), ctypes.c_float(0.125),
                                          buf.data_ptr() + 8192, 7, None, None, None) == 1
    # unknown q_layout: INVALID_ARG before any launch
    assert lib.veda_block_sparse_attn_fwd(plan.handle, buf.data_ptr(), 3, buf.data_ptr(), buf.data_ptr(),
                                          buf.data_ptr(), buf.data_ptr(), ctypes.c_float(0.125),
                                          buf.data_ptr() + 8192, 0, None, None, None) == 1
    assert "q_layout" in vb.veda_last_error()
    # q_perm NULL without the pooling workspace: INVALID_ARG
    assert lib.veda_permute_qkv(plan.handle, buf.data_ptr(), buf.data_ptr() + 4096, None, None,
                                buf.data_ptr() + 8192, None, None, 0, None) == 1
    assert lib.veda_score_tiles(plan.handle, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                                buf.data_ptr(), buf.data_ptr(), 16, None) == 4
    # the two-launch reductions refuse a short workspace (WORKSPACE) on the host
    short = plan.info["reduce_workspace_bytes"] - 16
    assert lib.veda_mask_mass(plan.handle, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                              buf.data_ptr(), short, None) == 4
    assert lib.veda_output_error(plan.handle, buf.data_ptr(), buf.data_ptr(), buf.data_ptr(), buf.data_ptr(),
                                 short, None) == 4
    # the backward refuses an output that aliases an input (INVALID_ARG), before any launch
    p_ = buf.data_ptr()
    assert lib.veda_block_sparse_attn_bwd(plan.handle, p_, p_ + 4096, p_ + 8192, p_ + 12288, p_ + 16384,
                                          p_ + 20480, p_, p_, p_, p_, ctypes.c_float(0.125), p_, p_ + 24576,
                                          p_ + 28672, p_ + 32768, 1 << 40, None) == 1
    assert lib.veda_block_sparse_attn_bwd(plan.handle, p_, p_ + 4096, p_ + 8192, p_ + 12288, p_ + 16384,
                                          p_ + 20480, p_, p_, p_, p_, ctypes.c_float(0.125), p_ + 24576,
                                          p_ + 24576, p_ + 28672, p_ + 32768, 1 << 40, None) == 1
    with pytest.raises(vb.VedaError):
        vb.veda_plan_upload(plan.handle, plan.tables)   # uploaded twice
