"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check_* function takes the oracle functions it checks as arguments, so the
mutation tests at the end can hand it a deliberately broken copy (a planted
mistake in the oracle, on the CPU) and show that the pin catches it.

Sources: Miowtion project page (intro "Sparse acceleration (Veda)", Key
Features > "Veda sparse attention"); "Deploying this checkpoint" (intro,
sections 0, 2 and 6); MiniMax-H3 cookbook page (heads, layers).
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import veda_oracle as vo
import veda_workloads as wl
from conftest import GOLDEN


# ---------------------------------------------------------------------------
# helpers (test side only)
# ---------------------------------------------------------------------------

def _read_tilings():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "tiling_small.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("grid"):
                g, t = line.split("|")
                grid = tuple(int(x) for x in g.split()[1:])
                tile = tuple(int(x) for x in t.split()[1:])
                cur = (grid, tile, [])
            elif line == "end":
                cases.append(cur)
            else:
                v, slots = line.split(":")
                cur[2].append((int(v), [int(x) for x in slots.split()]))
    return cases


def _small_partial_workload(heads=2, dim=64):
    """A grid with ragged edges on every axis: (4,10,12) with (2,8,8) tiles ->
    2x2x2 = 8 tiles, valid counts 128, 64, 32, 16 ..."""
    return wl.Workload(90, "small_partial", (wl.Segment(wl.VIDEO3D, (4, 10, 12), 0),),
                       heads, dim, ((2, 8, 8),) * heads, wl.KEEP_RATIO, 1, 4)


def _small_packed_workload():
    """Two video segments and a dense run, 64-aligned offsets."""
    segs = (wl.Segment(wl.VIDEO3D, (2, 8, 12), 0),
            wl.Segment(wl.VIDEO3D, (4, 10, 12), 192),
            wl.Segment(wl.DENSE1D, (1, 1, 200), 672))
    return wl.Workload(91, "small_packed", segs, 2, 64, ((2, 8, 8), (4, 4, 8)),
                       wl.KEEP_RATIO, 1, 3)


def _f64(t):
    return t.to(torch.float64).numpy()


def _random_bf16(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


_PLAN_CACHE = {}


def _plan(idx):
    if idx not in _PLAN_CACHE:
        _PLAN_CACHE[idx] = vo.Plan.from_workload(wl.workload(idx))
    return _PLAN_CACHE[idx]


# ---------------------------------------------------------------------------
# P1: tiling and permutation
# ---------------------------------------------------------------------------

def check_handworked_tilings(tiles_of_segment=vo.tiles_of_segment):
    for grid, tile, expected in _read_tilings():
        got = tiles_of_segment(vo.VIDEO3D, grid, 0, tile, 0)
        assert len(got) == len(expected), (grid, tile)
        for t, (valid, slots) in zip(got, expected):
            assert t.valid == valid, (grid, tile)
            assert t.tokens.tolist() == slots, (grid, tile, t.tokens.tolist(), slots)


def test_handworked_tilings():
    check_handworked_tilings()


def check_bijection(plan):
    for h in range(plan.num_heads):
        ht = plan.heads[h]
        perm = ht.perm()
        assert perm.shape[0] == ht.rows
        valid = perm[perm >= 0]
        assert np.array_equal(np.sort(valid), np.arange(plan.num_tokens))
        assert int(ht.valid_counts().sum()) == plan.num_tokens
        for i, t in enumerate(ht.tiles):
            assert 1 <= t.valid <= vo.TILE_TOKENS
            assert np.all(t.tokens[:t.valid] >= 0) and np.all(t.tokens[t.valid:] == -1)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_permutation_is_bijection(idx):
    check_bijection(_plan(idx))


def _hist(ht, segment=None):
    h = {}
    for t in ht.tiles:
        if segment is None or t.segment == segment:
            h[t.valid] = h.get(t.valid, 0) + 1
    return h


def test_valid_count_histograms():
    # worked by hand from the grid sizes (ragged last tile on each axis)
    assert _hist(_plan(1).heads[0]) == {128: 8}
    assert _hist(_plan(2).heads[0]) == {128: 64}
    assert _hist(_plan(3).heads[0]) == {128: 144, 96: 72, 72: 8}
    assert _hist(_plan(4).heads[0]) == {128: 840, 96: 120, 64: 84, 48: 12}
    assert _hist(_plan(4).heads[12]) == {128: 930, 32: 186}
    p5 = _plan(5).heads[0]
    assert _hist(p5, 0) == {128: 16}
    assert _hist(p5, 1) == {128: 144, 96: 72, 72: 8}
    assert _hist(p5, 2) == {128: 8}
    assert [p5.seg_count[s] for s in range(3)] == [16, 224, 8]


def test_identity_special_cases():
    # tile = whole grid of 128 tokens, and 1x1x128 rows of a width-128 grid
    seg = wl.Segment(wl.VIDEO3D, (2, 8, 8), 0)
    p = vo.Plan([seg], 1, 64, [(2, 8, 8)], vo.ALL_BLOCKS)
    assert np.array_equal(p.heads[0].perm(), np.arange(128))
    seg = wl.Segment(wl.VIDEO3D, (3, 2, 128), 0)
    p = vo.Plan([seg], 1, 64, [(1, 1, 128)], vo.ALL_BLOCKS)
    assert np.array_equal(p.heads[0].perm(), np.arange(768))
    seg = wl.Segment(wl.DENSE1D, (1, 1, 300), 64)
    p = vo.Plan([seg], 1, 64, [(2, 8, 8)], vo.ALL_BLOCKS)
    perm = p.heads[0].perm()
    assert perm[:300].tolist() == list(range(64, 364)) and np.all(perm[300:] == -1)


@pytest.mark.parametrize("idx", [1, 3, 5])
def test_inverse_of_forward_is_identity(idx):
    plan = _plan(idx)
    w = wl.workload(idx)
    x = _random_bf16((w.num_tokens, w.num_heads, 8), idx).view(torch.int16).numpy()
    y = vo.permute_forward(plan, x)
    assert y.shape == (plan.total_rows, 8)
    for h in range(plan.num_heads):
        perm = plan.heads[h].perm()
        pad = plan.row_offset[h] + np.nonzero(perm < 0)[0]
        assert np.all(y[pad] == 0)
    assert np.array_equal(vo.permute_inverse(plan, y), x)


# ---------------------------------------------------------------------------
# P2: pooling
# ---------------------------------------------------------------------------

def check_pool_special_cases(pool_tiles=vo.pool_tiles):
    w = _small_partial_workload(heads=1, dim=8)
    plan = vo.Plan.from_workload(w)
    ht = plan.heads[0]
    x = np.zeros((plan.total_rows, 8))
    # tile 0: constant; tile 1: a single distinct token, rest constant -3;
    # every partial tile: all values negative (padding zeros must not leak)
    for i, t in enumerate(ht.tiles):
        r0 = 128 * i
        x[r0:r0 + t.valid] = -1.5 - 0.25 * np.arange(t.valid)[:, None] - np.arange(8)[None, :]
    x[0:ht.tiles[0].valid] = 2.5
    f = pool_tiles(plan, x)
    assert np.all(f[0] == 2.5)
    for i, t in enumerate(ht.tiles):
        vals = x[128 * i:128 * i + t.valid]
        mx = vals.max(axis=0)
        mn = vals.min(axis=0)
        exact_mean = [Fraction(math.fsum(vals[:, d])) / t.valid for d in range(8)]
        assert np.array_equal(f[i, 8:16], mx.astype(np.float32)), i
        assert np.array_equal(f[i, 16:24], mn.astype(np.float32)), i
        for d in range(8):
            assert abs(Fraction(float(f[i, d])) - exact_mean[d]) <= abs(exact_mean[d]) * Fraction(1, 2 ** 24), (i, d)
        if t.valid < 128:
            assert np.all(f[i, 8:16] < 0), "padding leaked into max"


def test_pool_special_cases():
    check_pool_special_cases()


def test_pool_single_token_tile():
    seg = wl.Segment(wl.VIDEO3D, (1, 1, 129), 0)
    plan = vo.Plan([seg], 1, 4, [(1, 1, 128)], vo.ALL_BLOCKS)
    x = np.zeros((256, 4))
    x[128] = [3.0, -2.0, 0.5, 7.0]
    f = vo.pool_tiles(plan, x)
    assert f[1].tolist() == [3.0, -2.0, 0.5, 7.0] * 3


def test_pool_sum_is_exact_on_generated_inputs():
    """With the generator's flush, fp64 tile sums are exact: any order agrees."""
    w = wl.workload(2)
    inp = wl.make_inputs(w)
    plan = _plan(2)
    x = _f64(inp["q"])
    for h in range(2):
        perm = plan.heads[h].perm()
        for i in range(0, plan.heads[h].num_tiles, 7):
            toks = perm[128 * i:128 * i + plan.heads[h].tiles[i].valid]
            vals = x[toks, h]
            fwd = np.zeros(w.head_dim)
            for r in range(vals.shape[0]):
                fwd += vals[r]
            rev = np.zeros(w.head_dim)
            for r in range(vals.shape[0] - 1, -1, -1):
                rev += vals[r]
            assert np.array_equal(fwd, rev)
            assert all(Fraction(fwd[d]) == sum(Fraction(float(v)) for v in vals[:, d])
                       for d in range(0, w.head_dim, 31))


# ---------------------------------------------------------------------------
# P3: residual projection
# ---------------------------------------------------------------------------

def check_projection_one_hot(project=vo.project):
    plan = vo.Plan.from_workload(_small_partial_workload(heads=2, dim=8))
    D = 8
    rng = np.random.default_rng(0)
    feats = rng.standard_normal((plan.total_tiles, 3 * D)).astype(np.float32)
    mu, mx, mn = feats[:, :D], feats[:, D:2 * D], feats[:, 2 * D:]
    w0 = np.zeros((2, D, 3 * D), dtype=np.float32)
    assert np.array_equal(project(plan, feats, w0), mu), "W = 0 must give the mean"
    w1 = np.zeros_like(w0)
    for d in range(D):
        w1[0, d, D + d] = 1.0          # head 0: + max
        w1[1, d, 2 * D + ((d + 1) % D)] = 2.0   # head 1: + 2 min of the next channel
    got = project(plan, feats, w1)
    t0, t1 = plan.tile_offset[1], plan.tile_offset[2]
    exp0 = (mu[:t0].astype(np.float64) + mx[:t0]).astype(np.float32)
    exp1 = (mu[t0:t1].astype(np.float64) + 2.0 * np.roll(mn[t0:t1], -1, axis=1)).astype(np.float32)
    assert np.array_equal(got[:t0], exp0)
    assert np.array_equal(got[t0:t1], exp1)


def test_projection_one_hot():
    check_projection_one_hot()


def test_projection_matches_exact_rational_sum():
    w = wl.workload(1)
    inp = wl.make_inputs(w)
    plan = _plan(1)
    qp = vo.permute_forward(plan, _f64(inp["q"]))
    f = vo.pool_tiles(plan, qp)
    W = inp["w_q"].numpy()
    got = vo.project(plan, f, W)
    for h in range(2):
        for i in range(0, 8, 3):
            row = plan.tile_offset[h] + i
            for d in range(0, 64, 9):
                exact = Fraction(float(f[row, d])) + sum(
                    Fraction(float(W[h, d, e])) * Fraction(float(f[row, e])) for e in range(192))
                err = abs(Fraction(float(got[row, d])) - exact)
                assert err <= abs(exact) * Fraction(1, 2 ** 23) + Fraction(1, 2 ** 60)


# ---------------------------------------------------------------------------
# P4: pair scores
# ---------------------------------------------------------------------------

def check_score_orientation(score_pairs=vo.score_pairs):
    plan = vo.Plan.from_workload(_small_partial_workload(heads=1, dim=4))
    n = plan.total_tiles
    qh = np.zeros((n, 4), dtype=np.float32)
    kh = np.zeros((n, 4), dtype=np.float32)
    qh[:, 0] = np.arange(n)            # q_hat_i = (i, 1, 0, 0)
    qh[:, 1] = 1.0
    kh[:, 0] = 1.0                     # k_hat_j = (1, 10 j, 0, -0.5)
    kh[:, 1] = 10.0 * np.arange(n)
    kh[:, 3] = -0.5
    s = score_pairs(plan, qh, kh)[0]
    for i in range(n):
        for j in range(n):
            assert s[i, j] == np.float32(i + 10 * j), (i, j)
    # -0 is canonicalised to +0
    qz = np.zeros((n, 4), dtype=np.float32)
    qz[:, 0] = -1.0
    kz = np.zeros((n, 4), dtype=np.float32)
    s0 = score_pairs(plan, qz, kz)[0]
    assert not np.any(np.signbit(s0))


def test_score_orientation():
    check_score_orientation()


def test_scores_match_exact_rational_dot_products():
    w = wl.workload(1)
    inp = wl.make_inputs(w)
    plan = _plan(1)
    qh = vo.project(plan, vo.pool_tiles(plan, vo.permute_forward(plan, _f64(inp["q"]))), inp["w_q"].numpy())
    kh = vo.project(plan, vo.pool_tiles(plan, vo.permute_forward(plan, _f64(inp["k"]))), inp["w_k"].numpy())
    s = vo.score_pairs(plan, qh, kh)
    for h in range(2):
        for i in range(8):
            for j in range(8):
                a, b = plan.tile_offset[h] + i, plan.tile_offset[h] + j
                exact = sum(Fraction(float(qh[a, d])) * Fraction(float(kh[b, d])) for d in range(64))
                # the fp32 result is the exact value rounded (within half an fp32 ulp + fp64 noise)
                err = abs(Fraction(float(s[h][i, j])) - exact)
                assert err <= abs(exact) * Fraction(1, 2 ** 24) * Fraction(1001, 1000) + Fraction(1, 2 ** 70)


# ---------------------------------------------------------------------------
# P5: budgets
# ---------------------------------------------------------------------------

def _read_budgets():
    out = []
    with open(os.path.join(GOLDEN, "budgets.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, h, pair, rows, total, lo, nlo, hi, nhi = line.split()
                out.append((int(c), int(h), pair, int(rows), int(total), int(lo), int(nlo), int(hi), int(nhi)))
    return out


PAIR_SEGMENTS = {"AA": (0, 0), "RR": (0, 0), "RT": (0, 1), "TR": (1, 0), "TT": (1, 1)}


def check_golden_budgets(row_budgets=vo.row_budgets):
    for c, h, pair, rows, total, lo, nlo, hi, nhi in _read_budgets():
        plan = _plan(c)
        A, B = PAIR_SEGMENTS[pair]
        ht = plan.heads[h]
        k = row_budgets(plan, h)[ht.seg_first[A]:ht.seg_first[A] + ht.seg_count[A], B]
        assert len(k) == rows, (c, pair)
        assert int(k.sum()) == total, (c, pair, int(k.sum()), total)
        assert int((k == lo).sum()) == nlo and int((k == hi).sum()) == nhi, (c, pair)


def test_golden_budgets():
    check_golden_budgets()


def test_equal_kernel_cost_across_tile_shapes():
    plan = _plan(4)
    assert int(vo.row_budgets(plan, 0).sum()) == int(vo.row_budgets(plan, 23).sum()) == 95355


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_bresenham_invariants(idx):
    plan = _plan(idx)
    for h in sorted({0, plan.num_heads - 1}):
        ht = plan.heads[h]
        k = vo.row_budgets(plan, h)
        for A in range(len(plan.segments)):
            for B in range(len(plan.segments)):
                total = vo.pair_budget(plan, A, B)
                rows = k[ht.seg_first[A]:ht.seg_first[A] + ht.seg_count[A], B]
                if total is None:
                    assert np.all(rows == ht.seg_count[B])
                    continue
                b = total / ht.seg_count[A]
                assert int(rows.sum()) == vo.round_half_up(total) or A == B and b < 1
                prefix = 0
                for i, ki in enumerate(rows):
                    prefix += int(ki)
                    assert abs(prefix - (i + 1) * b) <= Fraction(1, 2)   # stays on the line
                    assert math.floor(b) <= ki <= math.floor(b) + 1


def test_budget_modes():
    w = wl.workload(1)
    plan = _plan(1)
    assert np.all(vo.row_budgets(plan, 0) == 2)
    pa = vo.Plan(w.segments, 2, 64, w.tile_shapes, vo.ALL_BLOCKS)
    assert np.all(vo.row_budgets(pa, 1) == 8)
    # a tiny keep ratio still keeps the diagonal; a huge fixed k is capped at n
    pk = vo.Plan(w.segments, 2, 64, w.tile_shapes, vo.KEEP_RATIO, 1, 1000)
    assert np.all(vo.row_budgets(pk, 0) == 1)
    pf = vo.Plan(w.segments, 2, 64, w.tile_shapes, vo.FIXED_K, fixed_k=50)
    assert np.all(vo.row_budgets(pf, 0) == 8)


def test_predictor_size_documentation_pin():
    vals = {}
    with open(os.path.join(GOLDEN, "predictor_size.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    D = vals["head_dim"]
    # the oracle's projection consumes [H, D, 3D] per map, two maps (q and k)
    plan = vo.Plan.from_workload(wl.workload(1))
    w = np.zeros((2, 64, 192), dtype=np.float32)
    assert vo.project(plan, np.zeros((16, 192), np.float32), w).shape == (16, 64)
    params = 2 * D * 3 * D * vals["heads"] * vals["layers"]
    assert params == 275_251_200
    assert round(params / 1e6) == vals["params_millions_printed"]
    # fp8 stores one byte per weight (262.5 MiB); the file also carries its tile plans
    assert vals["file_megabytes_printed"] - 1 <= params / 2 ** 20 <= vals["file_megabytes_printed"]


# ---------------------------------------------------------------------------
# P6: selection
# ---------------------------------------------------------------------------

def _brute_force_selected(s_row, cands, k, diag):
    """Rank counting (not sorting): j is kept iff fewer than k others beat it,
    where a beats b if its score is higher or equal with a lower index."""
    keep = set()
    if diag is not None:
        keep.add(diag)
        cands = [c for c in cands if c != diag]
        k -= 1
    for j in cands:
        beaten_by = sum(1 for c in cands if c != j and (s_row[c] > s_row[j] or (s_row[c] == s_row[j] and c < j)))
        if beaten_by < k:
            keep.add(j)
    return keep


def check_selection_brute_force(plan, scores, select_blocks=vo.select_blocks, heads=None):
    sel = select_blocks(plan, scores)
    for h in (range(plan.num_heads) if heads is None else heads):
        ht = plan.heads[h]
        k = vo.row_budgets(plan, h)
        for i, tile in enumerate(ht.tiles):
            row = sel[h][i]
            assert np.all(np.diff(row) > 0), "rows are sorted and unique"
            expect = set()
            for B in range(len(plan.segments)):
                cands = list(range(ht.seg_first[B], ht.seg_first[B] + ht.seg_count[B]))
                diag = i if tile.segment == B else None
                expect |= _brute_force_selected(scores[h][i], cands, int(k[i, B]), diag)
            assert set(row.tolist()) == expect, (h, i)
            assert i in expect or plan.segments[tile.segment].kind != vo.VIDEO3D


def _pipeline_scores(idx):
    w = wl.workload(idx)
    plan = _plan(idx)
    inp = wl.make_inputs(w)
    qh = vo.project(plan, vo.pool_tiles(plan, vo.permute_forward(plan, _f64(inp["q"]))), inp["w_q"].numpy())
    kh = vo.project(plan, vo.pool_tiles(plan, vo.permute_forward(plan, _f64(inp["k"]))), inp["w_k"].numpy())
    return plan, vo.score_pairs(plan, qh, kh)


def test_selection_brute_force_tiny():
    plan, scores = _pipeline_scores(1)
    check_selection_brute_force(plan, scores)


def test_selection_brute_force_grid():
    plan, scores = _pipeline_scores(2)
    check_selection_brute_force(plan, scores, heads=[0, 15])


def check_selection_ties(select_blocks=vo.select_blocks):
    w = _small_packed_workload()
    plan = vo.Plan.from_workload(w)
    rng = np.random.default_rng(3)
    scores = [rng.integers(-2, 3, size=(h.num_tiles, h.num_tiles)).astype(np.float32) for h in plan.heads]
    scores[0][:, :] = 0.0      # all ties on head 0: lowest indices win
    check_selection_brute_force(plan, scores, select_blocks)
    sel = select_blocks(plan, scores)
    ht = plan.heads[0]
    k = vo.row_budgets(plan, 0)
    i = ht.seg_first[1] + 5
    B = 1
    first = ht.seg_first[B]
    row_b = [j for j in sel[0][i] if first <= j < first + ht.seg_count[B]]
    exp = sorted({i} | set([j for j in range(first, first + ht.seg_count[B]) if j != i][:int(k[i, B]) - 1]))
    assert row_b == exp


def test_selection_ties():
    check_selection_ties()


def test_csr_packing():
    plan, scores = _pipeline_scores(1)
    sel = vo.select_blocks(plan, scores)
    rp, ci = vo.to_csr(plan, sel)
    assert rp.shape == (plan.total_tiles + 1,) and rp[-1] == ci.shape[0] == 32
    dm = vo.to_dense_mask(plan, sel)
    for h in range(2):
        for i in range(8):
            r = plan.tile_offset[h] + i
            assert np.array_equal(np.nonzero(dm[h][i])[0], ci[rp[r]:rp[r + 1]])
            assert dm[h][i, i] == 1


# ---------------------------------------------------------------------------
# P7: attention against the library's masked softmax attention
# ---------------------------------------------------------------------------

def _token_tile(plan, h, N):
    perm = plan.heads[h].perm()
    tile_of = np.empty(N, dtype=np.int64)
    slots = np.nonzero(perm >= 0)[0]
    tile_of[perm[slots]] = slots // 128
    return tile_of


def _sdpa_block_masked(plan, q, k, v, selection, scale):
    """Library masked attention over natural order: token a may see token b iff
    (tile(a), tile(b)) is a selected block of that head."""
    N, H, D = q.shape
    Os, Ls = np.zeros((N, H, D)), np.zeros((N, H))
    for h in range(H):
        tile_of = _token_tile(plan, h, N)
        n = plan.heads[h].num_tiles
        bm = np.zeros((n, n), dtype=bool)
        for i, r in enumerate(selection[h]):
            bm[i, r] = True
        m = torch.from_numpy(bm[tile_of][:, tile_of])
        qt = torch.from_numpy(np.ascontiguousarray(q[:, h]))
        kt = torch.from_numpy(np.ascontiguousarray(k[:, h]))
        vt = torch.from_numpy(np.ascontiguousarray(v[:, h]))
        o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=m[None], scale=scale)[0]
        logits = (scale * (qt @ kt.T.contiguous())).masked_fill(~m, float("-inf"))
        Os[:, h] = o.numpy()
        Ls[:, h] = torch.logsumexp(logits, dim=-1).numpy()
    return Os, Ls


def check_attention_vs_library(w, selection_kind, block_sparse_attention=vo.block_sparse_attention, seed=0):
    plan = vo.Plan.from_workload(w)
    N, H, D = w.num_tokens, w.num_heads, w.head_dim
    q = _f64(_random_bf16((N, H, D), seed))
    k = _f64(_random_bf16((N, H, D), seed + 1))
    v = _f64(_random_bf16((N, H, D), seed + 2))
    if selection_kind == "all":
        sel = vo.all_blocks_selection(plan)
    elif selection_kind == "diag":
        sel = [[np.array([i]) for i in range(plan.heads[h].num_tiles)] for h in range(H)]
    else:
        rng = np.random.default_rng(seed)
        sel = []
        for h in range(H):
            n = plan.heads[h].num_tiles
            sel.append([np.array(sorted({i} | set(rng.choice(n, size=rng.integers(1, n + 1), replace=False).tolist())))
                        for i in range(n)])
    scale = w.softmax_scale
    O, L = block_sparse_attention(plan, vo.permute_forward(plan, q), vo.permute_forward(plan, k),
                                  vo.permute_forward(plan, v), sel, scale)
    O_nat = vo.permute_inverse(plan, np.nan_to_num(O))
    L_nat = vo.permute_inverse(plan, np.nan_to_num(L)[:, None])[:, :, 0]
    if selection_kind == "all":
        Oref, Lref = vo.dense_attention(q, k, v, scale)
    else:
        Oref, Lref = _sdpa_block_masked(plan, q, k, v, sel, scale)
    assert np.max(np.abs(O_nat - Oref)) < 1e-10
    assert np.max(np.abs(L_nat - Lref)) < 1e-10
    # padded query rows stay undefined and never leak into valid rows
    for h in range(H):
        perm = plan.heads[h].perm()
        assert np.all(np.isnan(O[plan.row_offset[h] + np.nonzero(perm < 0)[0]]))


@pytest.mark.parametrize("kind", ["all", "diag", "random"])
def test_attention_vs_library_partial_tiles(kind):
    check_attention_vs_library(_small_partial_workload(), kind)


@pytest.mark.parametrize("kind", ["all", "random"])
def test_attention_vs_library_packed(kind):
    check_attention_vs_library(_small_packed_workload(), kind, seed=5)


def test_attention_vs_library_tiny_all():
    check_attention_vs_library(wl.workload(1), "all", seed=11)


def test_dense_reference_is_softmax():
    """The library route itself against an explicit fp64 softmax on 3 tokens."""
    q = np.array([[[1.0, 0.0]], [[0.0, 2.0]], [[1.0, 1.0]]])
    k = np.array([[[0.5, 0.5]], [[1.0, -1.0]], [[0.0, 3.0]]])
    v = np.array([[[1.0, 2.0]], [[3.0, 4.0]], [[5.0, 6.0]]])
    O, L = vo.dense_attention(q, k, v, 0.5)
    for a in range(3):
        z = [0.5 * (q[a, 0] @ k[b, 0]) for b in range(3)]
        e = [math.exp(x) for x in z]
        o = [sum(e[b] * v[b, 0, d] for b in range(3)) / sum(e) for d in range(2)]
        assert abs(L[a, 0] - math.log(sum(e))) < 1e-14
        assert np.allclose(O[a, 0], o, atol=1e-14)


# ---------------------------------------------------------------------------
# P8: block heat
# ---------------------------------------------------------------------------

def check_heat(w, block_heat=vo.block_heat, seed=7):
    plan = vo.Plan.from_workload(w)
    N, H, D = w.num_tokens, w.num_heads, w.head_dim
    q = _f64(_random_bf16((N, H, D), seed))
    k = _f64(_random_bf16((N, H, D), seed + 1))
    qp, kp = vo.permute_forward(plan, q), vo.permute_forward(plan, k)
    _, L = vo.block_sparse_attention(plan, qp, kp, kp, vo.all_blocks_selection(plan), w.softmax_scale)
    heat = block_heat(plan, qp, kp, L, w.softmax_scale)
    for h in range(H):
        assert np.allclose(heat[h].sum(axis=1), 1.0, atol=1e-12)
        # library softmax probabilities over natural order, averaged per block
        P = torch.softmax(w.softmax_scale * torch.from_numpy(q[:, h]) @ torch.from_numpy(k[:, h]).T, dim=-1).numpy()
        tile_of = _token_tile(plan, h, N)
        n = plan.heads[h].num_tiles
        ref = np.zeros((n, n))
        for i in range(n):
            rows = tile_of == i
            for j in range(n):
                ref[i, j] = P[rows][:, tile_of == j].sum() / rows.sum()
        assert np.max(np.abs(heat[h] - ref)) < 1e-12


def test_heat_partial_tiles():
    check_heat(_small_partial_workload())


def test_heat_packed():
    check_heat(_small_packed_workload())


def test_heat_row_subset():
    """block_heat restricted to some query tiles computes exactly those rows
    (pinned above against library softmax probabilities), reading the LSE of
    those rows only (NaN elsewhere), and leaves the other rows NaN."""
    w = _small_packed_workload()
    plan = vo.Plan.from_workload(w)
    N, H, D = w.num_tokens, w.num_heads, w.head_dim
    q = _f64(_random_bf16((N, H, D), 7))
    k = _f64(_random_bf16((N, H, D), 8))
    qp, kp = vo.permute_forward(plan, q), vo.permute_forward(plan, k)
    _, L = vo.block_sparse_attention(plan, qp, kp, kp, vo.all_blocks_selection(plan), w.softmax_scale)
    full = vo.block_heat(plan, qp, kp, L, w.softmax_scale)
    n = plan.heads[0].num_tiles
    rows = [0, n - 1]
    Lsub = np.full_like(L, np.nan)
    for i in rows:
        r0 = plan.row_offset[0] + 128 * i
        Lsub[r0:r0 + 128] = L[r0:r0 + 128]
    sub = vo.block_heat(plan, qp, kp, Lsub, w.softmax_scale, heads=[0], rows=rows)
    assert sub[1] is None if H > 1 else True
    for i in range(n):
        if i in rows:
            assert np.array_equal(sub[0][i], full[0][i])
        else:
            assert np.all(np.isnan(sub[0][i]))


# ---------------------------------------------------------------------------
# P10: attention mass of a mask, oracle mask, recall
# ---------------------------------------------------------------------------

def _heat_and_probs(w, seed=11):
    """Oracle heat of a workload and the token-level softmax probabilities
    (library softmax over natural order) it summarises."""
    plan = vo.Plan.from_workload(w)
    N, H, D = w.num_tokens, w.num_heads, w.head_dim
    q = _f64(_random_bf16((N, H, D), seed))
    k = _f64(_random_bf16((N, H, D), seed + 1))
    qp, kp = vo.permute_forward(plan, q), vo.permute_forward(plan, k)
    _, L = vo.block_sparse_attention(plan, qp, kp, kp, vo.all_blocks_selection(plan), w.softmax_scale)
    heat = vo.block_heat(plan, qp, kp, L, w.softmax_scale)
    probs = [torch.softmax(w.softmax_scale * torch.from_numpy(q[:, h]) @ torch.from_numpy(k[:, h]).T,
                           dim=-1).numpy() for h in range(H)]
    return plan, heat, probs


def check_mask_mass_token_level(mask_mass=vo.mask_mass):
    """Mass of a mask = mean over valid query tokens of the probability they
    put on the keys of their tile's kept key tiles, computed token by token."""
    w = _small_partial_workload()
    plan, heat, probs = _heat_and_probs(w)
    rng = np.random.default_rng(3)
    N = w.num_tokens
    sel = []
    for h in range(w.num_heads):
        n = plan.heads[h].num_tiles
        sel.append([np.sort(rng.choice(n, size=rng.integers(1, n + 1), replace=False)) for _ in range(n)])
    got = mask_mass(plan, heat, sel)
    for h in range(w.num_heads):
        tile_of = _token_tile(plan, h, N)
        kept = 0.0
        for r in range(N):
            keep_tiles = sel[h][tile_of[r]]
            kept += probs[h][r, np.isin(tile_of, keep_tiles)].sum()
        assert abs(got[h] - kept / N) < 1e-12, (h, got[h], kept / N)


def test_mask_mass_token_level():
    check_mask_mass_token_level()


def test_mask_mass_all_blocks_is_one():
    w = _small_packed_workload()
    plan, heat, _ = _heat_and_probs(w)
    m = vo.mask_mass(plan, heat, vo.all_blocks_selection(plan))
    assert np.allclose(m, 1.0, atol=1e-12)


def test_oracle_mask_is_best_under_the_budgets():
    """Brute force: per row, no choice of key tiles with the row's budget that
    contains the diagonal keeps more heat than the oracle mask; so the
    recall of any such mask (the predictor's) is at most 1."""
    w = _small_partial_workload()
    plan, heat, _ = _heat_and_probs(w)
    orc = vo.oracle_mask(plan, heat)
    rng = np.random.default_rng(5)
    scores = [rng.standard_normal(hm.shape) for hm in heat]
    pred = vo.select_blocks(plan, scores)
    for h in range(w.num_heads):
        n = plan.heads[h].num_tiles
        k = vo.row_budgets(plan, h).sum(axis=1)
        for i in range(n):
            best = max(heat[h][i, list(c)].sum() for c in itertools.combinations(range(n), int(k[i])) if i in c)
            assert abs(heat[h][i, orc[h][i]].sum() - best) < 1e-15
            assert len(orc[h][i]) == k[i] and i in orc[h][i]
    r = vo.recall(vo.mask_mass(plan, heat, pred), vo.mask_mass(plan, heat, orc))
    assert np.all(r <= 1.0 + 1e-15) and np.all(r > 0.0)


# ---------------------------------------------------------------------------
# P11: tile-plan search
# ---------------------------------------------------------------------------

def test_relative_output_error_closed_forms():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((50, 3, 8))
    eps = np.array([0.5, 0.1, 0.0])
    o = ref * (1.0 + eps)[None, :, None]
    assert np.allclose(vo.relative_output_error(o, ref), eps ** 2, rtol=1e-12, atol=1e-30)
    assert np.allclose(vo.relative_output_error(np.zeros_like(ref), ref), 1.0, rtol=1e-15)


_SEARCH_CANDIDATES = ((1, 8, 16), (2, 8, 8), (4, 4, 8))


def _frame_local_samples(n_samples=2, heads=2, dim=64):
    """q = k = a one-hot of the token's frame (t) plus small noise: attention
    stays inside each frame of a (4, 8, 16) grid."""
    segs = (wl.Segment(wl.VIDEO3D, (4, 8, 16), 0),)
    N = 512
    t_of = np.arange(N) // 128
    out = []
    for s in range(n_samples):
        g = np.random.default_rng(100 + s)
        base = np.zeros((N, heads, dim))
        base[np.arange(N), :, t_of] = 10.0
        q = _f64(torch.from_numpy(base + 0.05 * g.standard_normal((N, heads, dim))).to(torch.bfloat16))
        k = _f64(torch.from_numpy(base + 0.05 * g.standard_normal((N, heads, dim))).to(torch.bfloat16))
        v = _f64(torch.from_numpy(g.standard_normal((N, heads, dim))).to(torch.bfloat16))
        out.append((q, k, v))
    return segs, out


def check_search_prefers_frame_tiles(errors=vo.tile_plan_errors):
    """Attention confined to frames, two key tiles per row.  A (1, 8, 16)
    tile is a whole frame: its diagonal block already holds the mass.  A
    (2, 8, 8) tile is half of two frames: the diagonal plus the one other
    tile with the other halves (the heat picks it) hold the mass.  A (4, 4, 8)
    tile is a quarter of four frames and needs four blocks: large error."""
    segs, samples = _frame_local_samples()
    err = errors(segs, 2, 64, _SEARCH_CANDIDATES, wl.FIXED_K, 1, 10, 2, samples, 1.0 / 8.0)
    assert np.all(err[:, :2, :] < 1e-3), err[:, :2, :]
    assert np.all(err[:, 2, :] > 0.1), err[:, 2, :]
    assert set(vo.vote_tile_shapes(err).tolist()) <= {0, 1}


def test_search_prefers_frame_tiles():
    check_search_prefers_frame_tiles()


def test_search_all_blocks_has_no_error():
    segs, samples = _frame_local_samples(n_samples=1)
    err = vo.tile_plan_errors(segs, 2, 64, _SEARCH_CANDIDATES, wl.ALL_BLOCKS, 1, 10, 0, samples, 1.0 / 8.0)
    assert np.all(err < 1e-25), err


def test_vote_golden():
    """Hand-worked vote tables (every tie to the lower index)."""
    e = np.zeros((3, 4, 5))
    # per sample lowest error:   head0: c2,c2,c1  head1: c0,c1,c1  head2: c3,c3,c3
    #                            head3: c1,c2,c3 (one vote each -> c1)   head4: c0,c0,c2
    best = [[2, 0, 3, 1, 0], [2, 1, 3, 2, 0], [1, 1, 3, 3, 2]]
    for s in range(3):
        for h in range(5):
            e[s, :, h] = 1.0 + h + np.arange(4) * 0.01
            e[s, best[s][h], h] = 0.5
    # preferred: c2, c1, c3, c1, c0 -> heads per candidate: c0 1, c1 2, c2 1, c3 1
    # kept (2 shapes): c1 (2 heads), then c0 (tie of 1 head with c2, c3 -> lowest index)
    # heads 1, 3, 4 keep their preferred; heads 0 and 2 take the kept one with the lower mean error
    got = vo.vote_tile_shapes(e, max_shapes=2)
    # head 0 means: c0 = (1.0+1.0+1.0)/3 ... c1 = (1.01+1.01+0.5)/3 -> c1; head 2: c0 = 3.0, c1 = 3.01 -> c0
    assert np.array_equal(got, [1, 1, 0, 1, 0]), got
    assert np.array_equal(vo.vote_tile_shapes(e, max_shapes=4), [2, 1, 3, 1, 0])
    assert np.array_equal(vo.vote_tile_shapes(e, max_shapes=1), [1, 1, 1, 1, 1])


def test_vote_invariants_random():
    rng = np.random.default_rng(8)
    for _ in range(200):
        S, C, H = rng.integers(1, 5), rng.integers(1, 6), rng.integers(1, 9)
        e = rng.integers(0, 4, size=(S, C, H)).astype(np.float64)   # many ties
        for m in (1, 2, 3):
            out = vo.vote_tile_shapes(e, m)
            assert len(set(out.tolist())) <= m and np.all((out >= 0) & (out < C))
        # a head every sample agrees on, with at most two distinct such shapes, keeps its shape
        if S == 1 and len(set(np.argmin(e[0], axis=0).tolist())) <= 2:
            assert np.array_equal(vo.vote_tile_shapes(e, 2), np.argmin(e[0], axis=0))


# ---------------------------------------------------------------------------
# P12: block-sparse backward and transposed lists
# ---------------------------------------------------------------------------

def _random_selection(plan, seed):
    rng = np.random.default_rng(seed)
    sel = []
    for h in range(plan.num_heads):
        n = plan.heads[h].num_tiles
        sel.append([np.array(sorted({i} | set(rng.choice(n, size=rng.integers(1, n + 1), replace=False).tolist())))
                    for i in range(n)])
    return sel


def check_backward_vs_autograd(w, backward=vo.block_sparse_attention_backward, seed=3):
    """Gradients against torch autograd (fp64) of library masked attention over
    natural order, for a random upstream gradient dO."""
    plan = vo.Plan.from_workload(w)
    N, H, D = w.num_tokens, w.num_heads, w.head_dim
    q = _f64(_random_bf16((N, H, D), seed))
    k = _f64(_random_bf16((N, H, D), seed + 1))
    v = _f64(_random_bf16((N, H, D), seed + 2))
    do = _f64(_random_bf16((N, H, D), seed + 3))
    sel = _random_selection(plan, seed)
    scale = w.softmax_scale
    perm = lambda x: vo.permute_forward(plan, x)   # noqa: E731
    dQ, dK, dV = backward(plan, perm(q), perm(k), perm(v), perm(do), sel, scale)
    got = [vo.permute_inverse(plan, g) for g in (dQ, dK, dV)]
    for h in range(H):
        tile_of = _token_tile(plan, h, N)
        n = plan.heads[h].num_tiles
        bm = np.zeros((n, n), dtype=bool)
        for i, r in enumerate(sel[h]):
            bm[i, r] = True
        m = torch.from_numpy(bm[tile_of][:, tile_of])
        qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x[:, h])).requires_grad_(True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=m[None],
                                                             scale=scale)[0]
        o.backward(torch.from_numpy(np.ascontiguousarray(do[:, h])))
        for g, ref in zip(got, (qt.grad, kt.grad, vt.grad)):
            assert np.max(np.abs(g[:, h] - ref.numpy())) < 1e-10


def test_backward_vs_autograd_partial_tiles():
    check_backward_vs_autograd(_small_partial_workload())


def test_backward_vs_autograd_packed():
    check_backward_vs_autograd(_small_packed_workload())


def test_backward_padding_rows_are_zero():
    w = _small_partial_workload()
    plan = vo.Plan.from_workload(w)
    N, H, D = w.num_tokens, w.num_heads, w.head_dim
    xs = [vo.permute_forward(plan, _f64(_random_bf16((N, H, D), s))) for s in range(4)]
    dQ, dK, dV = vo.block_sparse_attention_backward(plan, *xs, _random_selection(plan, 1), w.softmax_scale)
    for h in range(H):
        pad = plan.row_offset[h] + np.nonzero(plan.heads[h].perm() < 0)[0]
        assert pad.size and not np.any(dQ[pad]) and not np.any(dK[pad]) and not np.any(dV[pad])


def test_mask_transpose_brute_force():
    w = _small_packed_workload()
    plan = vo.Plan.from_workload(w)
    sel = _random_selection(plan, 2)
    tr = vo.mask_transpose(plan, sel)
    for h in range(plan.num_heads):
        n = plan.heads[h].num_tiles
        for j in range(n):
            expect = [i for i in range(n) if j in set(sel[h][i].tolist())]
            assert tr[h][j].tolist() == expect
        assert sum(len(c) for c in tr[h]) == sum(len(r) for r in sel[h])


# ---------------------------------------------------------------------------
# Planted mistakes: each pin above must catch a plausible error in the oracle
# ---------------------------------------------------------------------------

def _mut_tiles_colmajor(kind, grid, offset, shape, si):
    """Valid box listed with x slowest instead of t slowest."""
    tiles = vo.tiles_of_segment(kind, grid, offset, shape, si)
    T, H, W = grid
    for t in tiles:
        v = t.tokens[:t.valid] - offset
        key = (v % W) * (T * H) + (v // W) % H * T + v // (W * H)
        t.tokens[:t.valid] = v[np.argsort(key)] + offset
    return tiles


def _mut_pool_divide_by_volume(plan, x):
    f = vo.pool_tiles(plan, x)
    D = x.shape[1]
    for h in range(plan.num_heads):
        for i, t in enumerate(plan.heads[h].tiles):
            f[plan.tile_offset[h] + i, :D] *= np.float32(t.valid / 128.0)
    return f


def _mut_pool_include_padding(plan, x):
    f = vo.pool_tiles(plan, x)
    D = x.shape[1]
    for h in range(plan.num_heads):
        for i, t in enumerate(plan.heads[h].tiles):
            if t.valid < 128:
                row = plan.tile_offset[h] + i
                f[row, D:2 * D] = np.maximum(f[row, D:2 * D], 0)
    return f


def _mut_project_transposed(plan, feats, w):
    D = w.shape[1]
    wt = np.zeros_like(w)
    wt[:, :, :D] = np.transpose(w[:, :, :D], (0, 2, 1))
    wt[:, :, D:2 * D] = np.transpose(w[:, :, D:2 * D], (0, 2, 1))
    wt[:, :, 2 * D:] = np.transpose(w[:, :, 2 * D:], (0, 2, 1))
    return vo.project(plan, feats, wt)


def _mut_project_feature_order(plan, feats, w):
    D = w.shape[1]
    f2 = feats.copy()
    f2[:, D:2 * D], f2[:, 2 * D:] = feats[:, 2 * D:], feats[:, D:2 * D]
    out = vo.project(plan, f2, w)
    return out


def _mut_scores_transposed(plan, qh, kh):
    return [s.T.copy() for s in vo.score_pairs(plan, qh, kh)]


def _mut_budget_floor(plan, h):
    k = vo.row_budgets(plan, h)
    ht = plan.heads[h]
    for A in range(len(plan.segments)):
        for B in range(len(plan.segments)):
            total = vo.pair_budget(plan, A, B)
            if total is None or plan.budget_mode != vo.KEEP_RATIO:
                continue
            b = total / ht.seg_count[A]
            for li in range(ht.seg_count[A]):
                ki = math.floor((li + 1) * b) - math.floor(li * b)
                if A == B:
                    ki = max(ki, 1)
                k[ht.seg_first[A] + li, B] = min(ki, ht.seg_count[B])
    return k


def _mut_select_ties_high(plan, scores):
    flipped = []
    for s in scores:
        n = s.shape[0]
        flipped.append(s[:, ::-1].copy())
    sel = vo.select_blocks(plan, flipped)
    out = []
    for h, rows in enumerate(sel):
        n = plan.heads[h].num_tiles
        out.append([np.array(sorted(n - 1 - r)) for r in rows])
    return out


def _mut_attention_no_padding_mask(plan, q_perm, k_perm, v_perm, selection, scale, rows=None):
    orig = plan.heads
    patched = []
    for ht in orig:
        tiles = [vo.Tile(t.segment, 128, t.tokens) for t in ht.tiles]
        patched.append(vo.HeadTiling(ht.shape, tiles, ht.seg_first, ht.seg_count))
    plan.heads = patched
    try:
        O, L = vo.block_sparse_attention(plan, q_perm, k_perm, v_perm, selection, scale, rows)
    finally:
        plan.heads = orig
    for h in range(plan.num_heads):   # keep padded query rows undefined as before
        perm = plan.heads[h].perm()
        pad = plan.row_offset[h] + np.nonzero(perm < 0)[0]
        O[pad] = np.nan
        L[pad] = np.nan
    return O, L


def _mut_heat_divide_by_volume(plan, q_perm, k_perm, lse, scale, heads=None):
    heat = vo.block_heat(plan, q_perm, k_perm, lse, scale, heads)
    for h, m in enumerate(heat):
        if m is not None:
            heat[h] = m * np.array([t.valid for t in plan.heads[h].tiles])[:, None] / 128.0
    return heat


def _mut_mass_unweighted(plan, heat, selection):
    out = np.zeros(plan.num_heads)
    for h in range(plan.num_heads):
        out[h] = np.mean([heat[h][i, r].sum() for i, r in enumerate(selection[h])])
    return out


def _mut_search_lowest_heat(segments, num_heads, head_dim, candidates, budget_mode, keep_num, keep_den, fixed_k,
                            samples, scale):
    """Takes the blocks of lowest heat as the best mask."""
    S, C, H = len(samples), len(candidates), num_heads
    err = np.zeros((S, C, H))
    for si, (q, k, v) in enumerate(samples):
        o_dense, _ = vo.dense_attention(q, k, v, scale)
        for ci, shape in enumerate(candidates):
            plan = vo.Plan(segments, H, head_dim, [tuple(shape)] * H, budget_mode, keep_num, keep_den, fixed_k)
            qp, kp, vp = (vo.permute_forward(plan, x) for x in (q, k, v))
            _, L = vo.block_sparse_attention(plan, qp, kp, vp, vo.all_blocks_selection(plan), scale)
            heat = vo.block_heat(plan, qp, kp, L, scale)
            o, _ = vo.block_sparse_attention(plan, qp, kp, vp, vo.oracle_mask(plan, [-x for x in heat]), scale)
            err[si, ci] = vo.relative_output_error(vo.permute_inverse(plan, np.nan_to_num(o)), o_dense)
    return err


def _mut_backward_no_rowsum(plan, q_perm, k_perm, v_perm, do_perm, selection, scale):
    """dS = P * dP (the rowsum(dO * O) term dropped)."""
    D = q_perm.shape[1]
    dQ, dK, dV = (np.zeros((plan.total_rows, D)) for _ in range(3))
    for h in range(plan.num_heads):
        ht = plan.heads[h]
        base = plan.row_offset[h]
        for i, row in enumerate(selection[h]):
            nq = ht.tiles[i].valid
            r0 = base + 128 * i
            q = q_perm[r0:r0 + nq]
            do = do_perm[r0:r0 + nq]
            kr = np.concatenate([base + 128 * int(j) + np.arange(ht.tiles[int(j)].valid) for j in row])
            K, V = k_perm[kr], v_perm[kr]
            z = scale * (q @ K.T)
            p = np.exp(z - z.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            ds = p * (do @ V.T)
            dQ[r0:r0 + nq] = scale * (ds @ K)
            np.add.at(dK, kr, scale * (ds.T @ q))
            np.add.at(dV, kr, p.T @ do)
    return dQ, dK, dV


MUTATIONS = [
    ("tiling order inside a tile", lambda: check_handworked_tilings(_mut_tiles_colmajor)),
    ("mean over the padded volume", lambda: check_pool_special_cases(_mut_pool_divide_by_volume)),
    ("padding leaks into max", lambda: check_pool_special_cases(_mut_pool_include_padding)),
    ("projection transposed", lambda: check_projection_one_hot(_mut_project_transposed)),
    ("features max/min swapped", lambda: check_projection_one_hot(_mut_project_feature_order)),
    ("scores transposed", lambda: check_score_orientation(_mut_scores_transposed)),
    ("budgets floored, not Bresenham", lambda: check_golden_budgets(_mut_budget_floor)),
    ("ties to the highest index", lambda: check_selection_ties(_mut_select_ties_high)),
    ("no padding mask on keys", lambda: check_attention_vs_library(_small_partial_workload(), "random",
                                                                  _mut_attention_no_padding_mask)),
    ("heat divided by 128", lambda: check_heat(_small_partial_workload(), _mut_heat_divide_by_volume)),
    ("mask mass not weighted by valid queries", lambda: check_mask_mass_token_level(_mut_mass_unweighted)),
    ("search mask of the lowest heat", lambda: check_search_prefers_frame_tiles(_mut_search_lowest_heat)),
    ("backward without the row-sum term", lambda: check_backward_vs_autograd(_small_partial_workload(),
                                                                           _mut_backward_no_rowsum)),
]


@pytest.mark.parametrize("name,run", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, run):
    with pytest.raises(AssertionError):
        run()
