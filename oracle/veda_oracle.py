"""Plain CPU oracle for the Veda block-sparse attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code, table or helper with the HIP library; it
re-derives the tiling, the budgets and the masks from the pages on its own.

Sources (all on the web pages this method is described on):
  * Miowtion project page, intro bullet "Sparse acceleration (Veda)": video
    tokens go into 3D tiles of 128 tokens, a small per-head predictor scores
    (query tile, key tile) pairs, only the top-scoring blocks are computed.
  * Miowtion project page, Key Features > "Veda sparse attention": up to two
    (t, h, w) tile shapes per layer, padded grids with valid-prefix tiles,
    segmented reference/target budgets; equal-kernel-cost budgets with
    Bresenham rounding and forced diagonal tiles; mean/max/min pooling with a
    per-head residual projection; teacher block heat from the dense LSE;
    singleton mask_mod with full/partial block lists.
  * "Deploying this checkpoint", section 2 (SM90 - Hopper): 128x128 forward
    tile that matches the 128-row query tiles, dense block mask packed into
    index lists; intro: attention visits 10% of the key tiles, per head.

Where the pages leave a step open this module takes one plain reading; each
function names the reading it implements (A1..A18 in the design notes of the
repository use the same numbering).

Precision: floating point is carried in fp64, except where a reading fixes a
narrower result type (pooled features, projections and scores are fp32 values
produced from fp64 accumulation, readings A8/A9).

Parity status: every function here is pinned by the CPU tests (invariants,
closed forms, brute force, textbook special cases computed by a library).  The
pages' own quality figures (mask recall on real trajectories) cannot be
reproduced on synthetic data and are parity unpinned.
"""

from __future__ import annotations

import dataclasses
from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

import numpy as np

VIDEO3D = 0
DENSE1D = 1
KEEP_RATIO = 0
FIXED_K = 1
ALL_BLOCKS = 2

TILE_TOKENS = 128   # tokens per tile (Miowtion page, "Sparse acceleration (Veda)": 3-D tiles of 128 tokens)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# ---------------------------------------------------------------------------
# O1-O3: tiles and the per-head permutation
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Tile:
    segment: int          # index of the segment the tile belongs to
    valid: int            # number of real tokens (the valid prefix length)
    tokens: np.ndarray    # int64 [tile_volume]: token index per slot, -1 = padding


def tiles_of_segment(kind: int, grid: Tuple[int, int, int], offset: int,
                     shape: Tuple[int, int, int], seg_index: int) -> List[Tile]:
    """Cut one segment into tiles (readings A1-A3).

    VIDEO3D: the (T, H, W) grid is padded up to whole (a, b, c) tiles.  Tiles
    are visited row-major over the tile grid (A1).  Inside a tile, the tokens
    of its valid sub-box are listed row-major in (t, h, w) (A2) and fill the
    first slots; the remaining slots are padding (A3, "valid-prefix tiles").
    DENSE1D (audio, not 3-D): consecutive runs of 128 tokens, the last one
    padded (A13).
    """
    T, H, W = grid
    tiles: List[Tile] = []
    if kind == DENSE1D:
        n = T * H * W
        for tau in range(ceil_div(n, TILE_TOKENS)):
            valid = min(TILE_TOKENS, n - TILE_TOKENS * tau)
            tok = np.full(TILE_TOKENS, -1, dtype=np.int64)
            tok[:valid] = offset + TILE_TOKENS * tau + np.arange(valid)
            tiles.append(Tile(seg_index, valid, tok))
        return tiles
    a, b, c = shape
    vol = a * b * c
    for ta in range(ceil_div(T, a)):
        for tb in range(ceil_div(H, b)):
            for tc in range(ceil_div(W, c)):
                vt = min(a, T - ta * a)
                vh = min(b, H - tb * b)
                vw = min(c, W - tc * c)
                tok = np.full(vol, -1, dtype=np.int64)
                s = 0
                for u in range(vt):
                    for v in range(vh):
                        for w in range(vw):
                            t_ = ta * a + u
                            y_ = tb * b + v
                            x_ = tc * c + w
                            tok[s] = offset + (t_ * H + y_) * W + x_
                            s += 1
                tiles.append(Tile(seg_index, vt * vh * vw, tok))
    return tiles


@dataclasses.dataclass
class HeadTiling:
    """All tiles of one head, segments in packed order (O2)."""
    shape: Tuple[int, int, int]
    tiles: List[Tile]
    seg_first: List[int]     # first tile index of each segment
    seg_count: List[int]     # number of tiles of each segment

    @property
    def num_tiles(self) -> int:
        return len(self.tiles)

    @property
    def rows(self) -> int:
        return TILE_TOKENS * len(self.tiles)

    def perm(self) -> np.ndarray:
        """Slot -> token table of this head, -1 for padding (O3)."""
        return np.concatenate([t.tokens for t in self.tiles])

    def valid_counts(self) -> np.ndarray:
        return np.array([t.valid for t in self.tiles], dtype=np.int64)


def tile_head(segments, shape) -> HeadTiling:
    tiles: List[Tile] = []
    first, count = [], []
    for si, seg in enumerate(segments):
        part = tiles_of_segment(seg.kind, tuple(seg.grid), seg.offset, tuple(shape), si)
        first.append(len(tiles))
        count.append(len(part))
        tiles.extend(part)
    return HeadTiling(tuple(shape), tiles, first, count)


class Plan:
    """Everything the method fixes before looking at the data (O1, O2, O8).

    segments: objects with .kind, .grid, .offset (packed order).
    tile_shapes: one (a, b, c) per head, each with a*b*c == 128, at most two
    distinct shapes per layer (Key Features > Veda sparse attention).
    """

    def __init__(self, segments, num_heads: int, head_dim: int,
                 tile_shapes: Sequence[Tuple[int, int, int]], budget_mode: int,
                 keep_num: int = 1, keep_den: int = 10, fixed_k: int = 0):
        assert len(tile_shapes) == num_heads
        for s in tile_shapes:
            assert s[0] * s[1] * s[2] == TILE_TOKENS, "a tile holds 128 tokens"
        assert len(set(map(tuple, tile_shapes))) <= 2, "at most two shapes per layer"
        self.segments = list(segments)
        self.num_heads = num_heads
        self.head_dim = head_dim
        self.tile_shapes = [tuple(s) for s in tile_shapes]
        self.budget_mode = budget_mode
        self.keep = Fraction(keep_num, keep_den)
        self.fixed_k = fixed_k
        cache = {}
        self.heads: List[HeadTiling] = []
        for s in self.tile_shapes:
            if s not in cache:
                cache[s] = tile_head(self.segments, s)
            self.heads.append(cache[s])
        self.row_offset = np.cumsum([0] + [h.rows for h in self.heads]).tolist()
        self.tile_offset = np.cumsum([0] + [h.num_tiles for h in self.heads]).tolist()
        self.num_tokens = sum(seg.grid[0] * seg.grid[1] * seg.grid[2]
                              for seg in self.segments)

    @classmethod
    def from_workload(cls, w) -> "Plan":
        return cls(w.segments, w.num_heads, w.head_dim, w.tile_shapes,
                   w.budget_mode, w.keep_num, w.keep_den, w.fixed_k)

    @property
    def total_rows(self) -> int:
        return self.row_offset[-1]

    @property
    def total_tiles(self) -> int:
        return self.tile_offset[-1]

    def segment_tokens(self, si: int) -> int:
        g = self.segments[si].grid
        return g[0] * g[1] * g[2]


# ---------------------------------------------------------------------------
# O4: permutation of Q/K/V into tile-major order and back
# ---------------------------------------------------------------------------

def permute_forward(plan: Plan, x: np.ndarray) -> np.ndarray:
    """[N, H, D] natural -> [sum_h L_h, D] head-major tile order (A4, A5).

    Padding slots hold +0.  Bit copy: works on any dtype (bf16 as int16 view).
    """
    N, H, D = x.shape
    out = np.zeros((plan.total_rows, D), dtype=x.dtype)
    for h in range(H):
        perm = plan.heads[h].perm()
        slots = np.nonzero(perm >= 0)[0]
        out[plan.row_offset[h] + slots] = x[perm[slots], h]
    return out


def permute_inverse(plan: Plan, y: np.ndarray, num_tokens: Optional[int] = None) -> np.ndarray:
    """[sum_h L_h, D] -> [N, H, D]: valid slots go back to their token; padding is dropped."""
    D = y.shape[1]
    N = plan.num_tokens if num_tokens is None else num_tokens
    out = np.zeros((N, plan.num_heads, D), dtype=y.dtype)
    for h in range(plan.num_heads):
        perm = plan.heads[h].perm()
        slots = np.nonzero(perm >= 0)[0]
        out[perm[slots], h] = y[plan.row_offset[h] + slots]
    return out


# ---------------------------------------------------------------------------
# O5-O7: the predictor (pool, residual projection, pair scores)
# ---------------------------------------------------------------------------

def pool_tiles(plan: Plan, x_perm: np.ndarray) -> np.ndarray:
    """Mean, max and min of every tile over its valid slots (A6, A8).

    x_perm: float values of the permuted tensor (bf16 upcast), [sum L_h, D].
    Returns fp32 [sum n_h, 3D] laid out [mean | max | min].
    The mean is fp32(fp64 sum / n) with the sum taken in fp64; max and min are
    exact.
    """
    D = x_perm.shape[1]
    out = np.zeros((plan.total_tiles, 3 * D), dtype=np.float32)
    for h in range(plan.num_heads):
        ht = plan.heads[h]
        for i, tile in enumerate(ht.tiles):
            r0 = plan.row_offset[h] + TILE_TOKENS * i
            rows = np.asarray(x_perm[r0:r0 + tile.valid], dtype=np.float64)
            total = rows.sum(axis=0)                 # fp64
            mean = total / np.float64(tile.valid)    # fp64 division
            row = plan.tile_offset[h] + i
            out[row, 0:D] = mean.astype(np.float32)
            out[row, D:2 * D] = rows.max(axis=0).astype(np.float32)
            out[row, 2 * D:3 * D] = rows.min(axis=0).astype(np.float32)
    return out


def project(plan: Plan, feats: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-head residual projection (A7): x_hat = mean + W_h . [mean; max; min].

    w: fp32 [H, D, 3D].  For each output channel d the sum starts at the mean
    and adds W[h, d, e] * f[e] for e = 0 .. 3D-1 in ascending order, in fp64
    (each product of two fp32 values is exact in fp64); the result is rounded
    once to fp32.
    """
    H, D, E = w.shape
    out = np.zeros((plan.total_tiles, D), dtype=np.float32)
    for h in range(H):
        t0, t1 = plan.tile_offset[h], plan.tile_offset[h + 1]
        f = feats[t0:t1].astype(np.float64)          # [n, 3D]
        wh = w[h].astype(np.float64)                 # [D, 3D]
        acc = f[:, 0:D].copy()                       # residual: the mean
        for e in range(E):
            acc += f[:, e:e + 1] * wh[:, e][None, :]
        out[t0:t1] = acc.astype(np.float32)
    return out


def score_pairs(plan: Plan, q_hat: np.ndarray, k_hat: np.ndarray) -> List[np.ndarray]:
    """Pair scores s[i, j] = q_hat_i . k_hat_j per head (A9).

    fp64 sum over d = 0 .. D-1 in ascending order, rounded once to fp32;
    -0.0 is replaced by +0.0.  Returns one fp32 [n_h, n_h] array per head
    (row = query tile, column = key tile).
    """
    out = []
    D = q_hat.shape[1]
    for h in range(plan.num_heads):
        t0, t1 = plan.tile_offset[h], plan.tile_offset[h + 1]
        qh = q_hat[t0:t1].astype(np.float64)
        kh = k_hat[t0:t1].astype(np.float64)
        acc = np.zeros((t1 - t0, t1 - t0), dtype=np.float64)
        for d in range(D):
            acc += qh[:, d:d + 1] * kh[:, d][None, :]
        s = acc.astype(np.float32)
        s[s == 0] = np.float32(0.0)                  # -0 -> +0
        out.append(s)
    return out


# ---------------------------------------------------------------------------
# O8: budgets
# ---------------------------------------------------------------------------

def round_half_up(x: Fraction) -> int:
    """R(x) = floor(x + 1/2) for x >= 0."""
    return (2 * x.numerator + x.denominator) // (2 * x.denominator)


def pair_budget(plan: Plan, seg_a: int, seg_b: int) -> Optional[Fraction]:
    """Total blocks of a (query segment, key segment) pair, or None if the pair is dense.

    Equal kernel cost (A10): keep * (N_A / 128) * (N_B / 128) blocks, i.e. the
    keep ratio of what a dense kernel over the valid tokens would compute, so
    heads with different tile shapes or padding get the same block count.
    Pairs with a non-video segment are dense (A13).
    """
    if plan.budget_mode == ALL_BLOCKS:
        return None
    if plan.segments[seg_a].kind != VIDEO3D or plan.segments[seg_b].kind != VIDEO3D:
        return None
    na = plan.segment_tokens(seg_a)
    nb = plan.segment_tokens(seg_b)
    return plan.keep * Fraction(na * nb, TILE_TOKENS * TILE_TOKENS)


def row_budgets(plan: Plan, h: int) -> np.ndarray:
    """k[i, B]: blocks row i of head h takes from key segment B (A10-A12, A15).

    KEEP_RATIO: the pair total is spread over the query rows of segment A by
    midpoint Bresenham, k_i = R((i+1) b) - R(i b) with b = total / n_A.
    FIXED_K: k_i = fixed_k.  The diagonal is counted inside k_i (at least 1
    when A == B), and k_i never exceeds n_B.  Dense pairs take all of B.
    """
    ht = plan.heads[h]
    S = len(plan.segments)
    k = np.zeros((ht.num_tiles, S), dtype=np.int64)
    for A in range(S):
        nA = ht.seg_count[A]
        for B in range(S):
            nB = ht.seg_count[B]
            total = pair_budget(plan, A, B)
            for li in range(nA):
                if total is None:
                    ki = nB
                else:
                    if plan.budget_mode == FIXED_K:
                        ki = plan.fixed_k
                    else:
                        b = total / nA
                        ki = round_half_up((li + 1) * b) - round_half_up(li * b)
                    if A == B:
                        ki = max(ki, 1)
                    ki = min(ki, nB)
                k[ht.seg_first[A] + li, B] = ki
    return k


# ---------------------------------------------------------------------------
# O9: block selection
# ---------------------------------------------------------------------------

def select_blocks(plan: Plan, scores: List[np.ndarray]) -> List[List[np.ndarray]]:
    """Selected key tiles of every query tile, per head (A12-A15).

    For row i in segment A and each key segment B: the diagonal first when
    A == B, then B's remaining tiles in the order (score descending, key tile
    index ascending) until the row's budget for B is used.  Dense pairs take
    every tile of B.  Each row is returned sorted ascending.
    """
    result = []
    for h in range(plan.num_heads):
        ht = plan.heads[h]
        s = scores[h]
        assert np.all(np.isfinite(s)), "scores must be finite"
        k = row_budgets(plan, h)
        rows = []
        for i, tile in enumerate(ht.tiles):
            A = tile.segment
            chosen: List[int] = []
            for B in range(len(plan.segments)):
                first, count = ht.seg_first[B], ht.seg_count[B]
                kib = int(k[i, B])
                cands = list(range(first, first + count))
                if kib == count:
                    chosen.extend(cands)
                    continue
                if A == B:
                    chosen.append(i)
                    cands.remove(i)
                    kib -= 1
                order = sorted(cands, key=lambda j: (-float(s[i, j]), j))
                chosen.extend(order[:kib])
            rows.append(np.array(sorted(chosen), dtype=np.int64))
        result.append(rows)
    return result


def to_csr(plan: Plan, selection: List[List[np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Pack the mask into CSR over all rows of all heads (the pages' index lists).

    row_ptr int32 [sum n_h + 1]; col_idx int32 [nnz] holds head-local key
    tile indices, ascending within a row.
    """
    counts = [len(r) for rows in selection for r in rows]
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col = np.concatenate([r for rows in selection for r in rows]) if counts else np.zeros(0)
    return row_ptr.astype(np.int32), col.astype(np.int32)


def to_dense_mask(plan: Plan, selection: List[List[np.ndarray]]) -> List[np.ndarray]:
    out = []
    for h, rows in enumerate(selection):
        n = plan.heads[h].num_tiles
        m = np.zeros((n, n), dtype=np.uint8)
        for i, r in enumerate(rows):
            m[i, r] = 1
        out.append(m)
    return out


def all_blocks_selection(plan: Plan) -> List[List[np.ndarray]]:
    return [[np.arange(plan.heads[h].num_tiles, dtype=np.int64)
             for _ in range(plan.heads[h].num_tiles)] for h in range(plan.num_heads)]


# ---------------------------------------------------------------------------
# O10: block-sparse attention over the selected blocks
# ---------------------------------------------------------------------------

def attention_row_tile(plan: Plan, h: int, i: int, q_perm, k_perm, v_perm,
                       cols: Sequence[int], scale: float):
    """Masked softmax attention of the valid queries of tile i over the valid
    keys of the selected key tiles (A14, A17), in fp64.

    Returns (O [valid_i, D] fp64, LSE [valid_i] fp64, natural log).
    """
    ht = plan.heads[h]
    base = plan.row_offset[h]
    nq = ht.tiles[i].valid
    q = np.asarray(q_perm[base + TILE_TOKENS * i: base + TILE_TOKENS * i + nq], dtype=np.float64)
    ks, vs = [], []
    for j in cols:
        nk = ht.tiles[j].valid
        r0 = base + TILE_TOKENS * j
        ks.append(np.asarray(k_perm[r0:r0 + nk], dtype=np.float64))
        vs.append(np.asarray(v_perm[r0:r0 + nk], dtype=np.float64))
    K = np.concatenate(ks)
    V = np.concatenate(vs)
    z = scale * (q @ K.T)
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ V) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def block_sparse_attention(plan: Plan, q_perm, k_perm, v_perm,
                           selection: List[List[np.ndarray]], scale: float,
                           rows: Optional[Sequence[Tuple[int, int]]] = None):
    """O10 over whole heads (or a subset of (head, query tile) rows).

    Returns O fp64 [sum L_h, D] and LSE fp64 [sum L_h]; padded query rows
    (undefined, A5) and rows not computed are NaN.
    """
    D = q_perm.shape[1]
    O = np.full((plan.total_rows, D), np.nan)
    L = np.full(plan.total_rows, np.nan)
    if rows is None:
        rows = [(h, i) for h in range(plan.num_heads) for i in range(plan.heads[h].num_tiles)]
    for h, i in rows:
        o, lse = attention_row_tile(plan, h, i, q_perm, k_perm, v_perm, selection[h][i], scale)
        r0 = plan.row_offset[h] + TILE_TOKENS * i
        O[r0:r0 + o.shape[0]] = o
        L[r0:r0 + o.shape[0]] = lse
    return O, L


# ---------------------------------------------------------------------------
# O15: block-sparse attention backward, per-key-tile lists
# ---------------------------------------------------------------------------

def mask_transpose(plan: Plan, selection: List[List[np.ndarray]]) -> List[List[np.ndarray]]:
    """The transposed lists (reading A22): for every head and key tile j, the
    query tiles whose rows selected j, ascending."""
    out = []
    for h in range(plan.num_heads):
        n = plan.heads[h].num_tiles
        cols: List[List[int]] = [[] for _ in range(n)]
        for i, row in enumerate(selection[h]):
            for j in row:
                cols[int(j)].append(i)
        out.append([np.array(c, dtype=np.int64) for c in cols])
    return out


def block_sparse_attention_backward(plan: Plan, q_perm, k_perm, v_perm, do_perm,
                                    selection: List[List[np.ndarray]], scale: float):
    """Gradients of the masked softmax attention O10 (reading A22; Miowtion
    project page: the block-sparse backward the predictor and LoRA training
    need), in fp64, by the textbook softmax backward per query tile row:
      P = softmax(scale q K^T) over the valid keys of the selected tiles,
      dV += P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
      dQ = scale dS K,  dK += scale dS^T Q.
    Padded query rows and padding keys carry no gradient (zero rows).

    q/k/v/do_perm: [sum L_h, D].  Returns dQ, dK, dV fp64 [sum L_h, D].
    """
    D = q_perm.shape[1]
    dQ = np.zeros((plan.total_rows, D))
    dK = np.zeros((plan.total_rows, D))
    dV = np.zeros((plan.total_rows, D))
    for h in range(plan.num_heads):
        ht = plan.heads[h]
        base = plan.row_offset[h]
        for i, row in enumerate(selection[h]):
            nq = ht.tiles[i].valid
            r0 = base + TILE_TOKENS * i
            q = np.asarray(q_perm[r0:r0 + nq], dtype=np.float64)
            do = np.asarray(do_perm[r0:r0 + nq], dtype=np.float64)
            krows = np.concatenate([base + TILE_TOKENS * int(j) + np.arange(ht.tiles[int(j)].valid) for j in row])
            K = np.asarray(k_perm[krows], dtype=np.float64)
            V = np.asarray(v_perm[krows], dtype=np.float64)
            z = scale * (q @ K.T)
            p = np.exp(z - z.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            o = p @ V
            dp = do @ V.T
            ds = p * (dp - np.sum(do * o, axis=1, keepdims=True))
            dQ[r0:r0 + nq] = scale * (ds @ K)
            np.add.at(dK, krows, scale * (ds.T @ q))
            np.add.at(dV, krows, p.T @ do)
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# O11: block heat from the dense LSE
# ---------------------------------------------------------------------------

def block_heat(plan: Plan, q_perm, k_perm, lse: np.ndarray, scale: float,
               heads: Optional[Sequence[int]] = None,
               rows: Optional[Sequence[int]] = None) -> List[Optional[np.ndarray]]:
    """Teacher block heat (A16): heat[i, j] = mean over the valid queries r of
    tile i of the attention probability mass on the valid keys of tile j,
    exp(scale q_r.k_c - LSE_r) summed over c, with LSE the dense attention's
    log-sum-exp over all valid keys.  Each row is a distribution.  `rows`
    restricts the work to those query tiles of each head (the other rows of
    the returned matrices are NaN); only their LSE entries are read.
    """
    out: List[Optional[np.ndarray]] = [None] * plan.num_heads
    heads = range(plan.num_heads) if heads is None else heads
    for h in heads:
        ht = plan.heads[h]
        base = plan.row_offset[h]
        n = ht.num_tiles
        Kall = np.asarray(k_perm[base:base + ht.rows], dtype=np.float64)
        valid = ht.valid_counts()
        heat = np.zeros((n, n), dtype=np.float64)
        if rows is not None:
            heat[:] = np.nan
        for i in (range(n) if rows is None else rows):
            nq = int(valid[i])
            r0 = base + TILE_TOKENS * i
            q = np.asarray(q_perm[r0:r0 + nq], dtype=np.float64)
            p = np.exp(scale * (q @ Kall.T) - np.asarray(lse[r0:r0 + nq], dtype=np.float64)[:, None])
            for j in range(n):
                c0 = TILE_TOKENS * j
                heat[i, j] = p[:, c0:c0 + int(valid[j])].sum() / nq
        out[h] = heat
    return out


# ---------------------------------------------------------------------------
# O13: attention mass of a mask and recall against the oracle mask
# ---------------------------------------------------------------------------

def mask_mass(plan: Plan, heat: List[np.ndarray], selection: List[List[np.ndarray]]) -> np.ndarray:
    """Fraction of each head's attention probability mass that a mask keeps
    (reading A19): over the valid queries r of the head,
    sum_r sum_{j in mask(tile(r))} P(keys of tile j | r) / #valid queries.
    With heat[i, j] the mean of that inner sum over the valid queries of tile
    i (O11), this is sum_i nq_i * sum_{j in mask_i} heat[i, j] / sum_i nq_i.
    The "Deploying this checkpoint" page, section 6, quotes this quantity for
    the oracle mask; section 4 names recall against the oracle mask.

    heat: per head [n, n] (fp32 or fp64 values); returns fp64 [num_heads].
    """
    out = np.zeros(plan.num_heads, dtype=np.float64)
    for h in range(plan.num_heads):
        nq = plan.heads[h].valid_counts().astype(np.float64)
        hm = np.asarray(heat[h], dtype=np.float64)
        kept = 0.0
        for i, row in enumerate(selection[h]):
            kept += nq[i] * float(np.sum(hm[i, np.asarray(row, dtype=np.int64)]))
        out[h] = kept / float(np.sum(nq))
    return out


def oracle_mask(plan: Plan, heat: List[np.ndarray]) -> List[List[np.ndarray]]:
    """The oracle mask (A20): the same budgeted selection as the predictor's
    (forced diagonal, per-row budgets, ties to the lowest key tile) applied to
    the block heat instead of the predicted scores."""
    return select_blocks(plan, heat)


def recall(pred_mass: np.ndarray, oracle_mass: np.ndarray) -> np.ndarray:
    """Recall of a predicted mask: its attention mass over the oracle mask's."""
    return np.asarray(pred_mass, dtype=np.float64) / np.asarray(oracle_mass, dtype=np.float64)


# ---------------------------------------------------------------------------
# O14: tile-plan search (relative output error under the best mask, vote)
# ---------------------------------------------------------------------------

def relative_output_error(o: np.ndarray, o_ref: np.ndarray) -> np.ndarray:
    """Per head: sum over tokens and channels of (o - o_ref)^2 over the sum of
    o_ref^2 (the relative output MSE of reading A21).  o, o_ref: [N, H, D]."""
    d = np.asarray(o, dtype=np.float64) - np.asarray(o_ref, dtype=np.float64)
    r = np.asarray(o_ref, dtype=np.float64)
    return np.einsum("nhd,nhd->h", d, d) / np.einsum("nhd,nhd->h", r, r)


def tile_plan_errors(segments, num_heads: int, head_dim: int, candidates, budget_mode: int, keep_num: int,
                     keep_den: int, fixed_k: int, samples, scale: float) -> np.ndarray:
    """Oracle tile-plan search, error table (reading A21; Miowtion project
    page, Key Features: oracle tile-plan search by relative output MSE under
    the best mask).  For every sample s (q, k, v fp64 [N, H, D]) and
    candidate tile shape c (used by every head): the best mask is the oracle
    mask (top-k of the dense-LSE block heat under the budgets, O13), the
    sparse output is attention over it, and err[s, c, h] is its relative
    output error against dense attention over all tokens."""
    S, C, H = len(samples), len(candidates), num_heads
    err = np.zeros((S, C, H), dtype=np.float64)
    for si, (q, k, v) in enumerate(samples):
        o_dense, _ = dense_attention(q, k, v, scale)
        for ci, shape in enumerate(candidates):
            plan = Plan(segments, H, head_dim, [tuple(shape)] * H, budget_mode, keep_num, keep_den, fixed_k)
            qp, kp, vp = permute_forward(plan, q), permute_forward(plan, k), permute_forward(plan, v)
            _, L = block_sparse_attention(plan, qp, kp, vp, all_blocks_selection(plan), scale)
            heat = block_heat(plan, qp, kp, L, scale)
            o, _ = block_sparse_attention(plan, qp, kp, vp, oracle_mask(plan, heat), scale)
            err[si, ci] = relative_output_error(permute_inverse(plan, np.nan_to_num(o)), o_dense)
    return err


def vote_tile_shapes(err: np.ndarray, max_shapes: int = 2) -> np.ndarray:
    """Majority vote over samples, at most `max_shapes` shapes per layer
    (reading A21).  err [S, C, H] -> candidate index per head.

    1. Each sample votes, per head, for its lowest-error candidate.
    2. A head's preferred candidate is the one with the most votes.
    3. The layer keeps the `max_shapes` candidates preferred by the most heads.
    4. A head whose preferred candidate is kept uses it; any other head uses
       the kept candidate with the lowest mean error over the samples.
    Every tie goes to the lower candidate index.
    """
    S, C, H = err.shape
    votes = np.zeros((C, H), dtype=np.int64)
    for s in range(S):
        for h in range(H):
            votes[int(np.argmin(err[s, :, h])), h] += 1
    pref = np.array([int(np.argmax(votes[:, h])) for h in range(H)], dtype=np.int64)
    heads_for = np.bincount(pref, minlength=C)
    order = sorted(range(C), key=lambda c: (-heads_for[c], c))
    kept = [c for c in order[:max_shapes] if heads_for[c] > 0]
    mean = err.mean(axis=0)
    out = np.empty(H, dtype=np.int64)
    for h in range(H):
        if pref[h] in kept:
            out[h] = pref[h]
        else:
            out[h] = min(kept, key=lambda c: (mean[c, h], c))
    return out


# ---------------------------------------------------------------------------
# O12: dense attention over natural order, by a library routine
# ---------------------------------------------------------------------------

def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """softmax(scale Q K^T) V over all tokens of each head, by torch's
    scaled_dot_product_attention in fp64; LSE by torch.logsumexp.

    q, k, v: float [N, H, D].  Returns (O [N, H, D], LSE [N, H]) fp64.
    """
    import torch
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64)).permute(1, 0, 2).contiguous()
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(np.asarray(v, dtype=np.float64)).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt.unsqueeze(0), kt.unsqueeze(0), vt.unsqueeze(0), scale=scale)[0]
    lse = torch.logsumexp(scale * torch.matmul(qt, kt.transpose(1, 2).contiguous()), dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


# ---------------------------------------------------------------------------
# The whole path, end to end (used by the smoke check and the CPU baseline)
# ---------------------------------------------------------------------------

def bf16_to_f64(x) -> np.ndarray:
    """bf16 tensor (torch) -> fp64 numpy, exactly."""
    import torch
    return x.to(torch.float64).numpy()


def run_path(plan: Plan, q, k, v, w_q, w_k, scale: float, rows=None):
    """Permute, score, select, attend, unpermute.  q/k/v: fp64 numpy [N, H, D]
    holding bf16 values; w_q/w_k: fp32 numpy [H, D, 3D]."""
    qp = permute_forward(plan, q)
    kp = permute_forward(plan, k)
    vp = permute_forward(plan, v)
    fq = pool_tiles(plan, qp)
    fk = pool_tiles(plan, kp)
    qh = project(plan, fq, w_q)
    kh = project(plan, fk, w_k)
    scores = score_pairs(plan, qh, kh)
    sel = select_blocks(plan, scores)
    O, L = block_sparse_attention(plan, qp, kp, vp, sel, scale, rows=rows)
    return {"q_perm": qp, "k_perm": kp, "v_perm": vp, "feat_q": fq, "feat_k": fk,
            "q_hat": qh, "k_hat": kh, "scores": scores, "selection": sel,
            "o_perm": O, "lse": L}
