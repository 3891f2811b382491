"""Seeded synthetic workloads for the Veda sparse-attention hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds the five workload descriptions and the random-number
recipe that fills them, and nothing of the method itself: no tiling, pooling,
scoring, budgeting, selection or attention arithmetic lives here.

The workloads stand in for the MiniMax-H3 activations that the pages measure on
(the Miowtion project page, "Sparse acceleration (Veda)" and "Key Features";
"Deploying this checkpoint", section 6): the real trajectories and weights are
not available, so Q/K/V are Gaussian noise plus a smooth positional bias that
gives the scores the spatial locality real video attention has.

Locality bias: random Fourier features of an RBF kernel (Rahimi and Recht,
"Random Features for Large-Scale Kernel Machines", NIPS 2007).  Per head,
b(p)[2f] = a*cos(w_f . p) and b(p)[2f+1] = a*sin(w_f . p) with p = (t, y, x) the
token's position in its own segment grid, so b(p).b(p') approximates
a^2 F exp(-|(p-p')/l|^2 / 2).  The same b is added to Q and K of a head.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch

VIDEO3D = 0
DENSE1D = 1

KEEP_RATIO = 0
FIXED_K = 1
ALL_BLOCKS = 2

# Values below this magnitude are flushed to zero before the bf16 rounding.
# With it every non-zero bf16 input is a multiple of 2**-31, so a sum of 128 of
# them (magnitude < 2**10) is exact in fp64 whatever the summation order.
FLUSH_BELOW = 2.0 ** -24


@dataclasses.dataclass(frozen=True)
class Segment:
    """One segment of the packed token sequence, in natural (packed) order.

    kind:   VIDEO3D (a (t, h, w) latent grid) or DENSE1D (a 1-D run, e.g. audio).
    grid:   (T, H, W); a DENSE1D segment of length n is (1, 1, n).
    offset: index of the segment's first token in the packed sequence.
    """

    kind: int
    grid: Tuple[int, int, int]
    offset: int

    @property
    def length(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]


@dataclasses.dataclass(frozen=True)
class Workload:
    """A synthetic attention-layer workload."""

    index: int
    name: str
    segments: Tuple[Segment, ...]
    num_heads: int
    head_dim: int
    tile_shapes: Tuple[Tuple[int, int, int], ...]   # one (a, b, c) per head
    budget_mode: int
    keep_num: int = 1
    keep_den: int = 10
    fixed_k: int = 0
    locality_bias: bool = True
    with_heat: bool = False

    @property
    def num_tokens(self) -> int:
        return sum(s.length for s in self.segments)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def describe(self) -> str:
        segs = "+".join(
            ("%dx%dx%d" % s.grid) if s.kind == VIDEO3D else ("1d%d" % s.length)
            for s in self.segments)
        shapes = sorted(set(self.tile_shapes))
        return "%s: %s tokens=%d H=%d D=%d tiles=%s" % (
            self.name, segs, self.num_tokens, self.num_heads, self.head_dim,
            ",".join("%dx%dx%d" % t for t in shapes))


def _video(grid, offset=0):
    return Segment(VIDEO3D, tuple(grid), offset)


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny", (_video((4, 16, 16)),), 2, 64, ((2, 8, 8),) * 2,
                FIXED_K, fixed_k=2, locality_bias=False),
    2: Workload(2, "grid_8x32x32", (_video((8, 32, 32)),), 16, 128,
                ((4, 4, 8),) * 16, KEEP_RATIO),
    3: Workload(3, "clip16x9_16x30x54", (_video((16, 30, 54)),), 24, 128,
                ((2, 8, 8),) * 24, KEEP_RATIO),
    # Two tile shapes in one layer: heads 0-11 use (4,4,8), heads 12-23 use (1,8,16).
    4: Workload(4, "long_clip_31x48x84", (_video((31, 48, 84)),), 24, 128,
                ((4, 4, 8),) * 12 + ((1, 8, 16),) * 12, KEEP_RATIO),
    # Packed reference + target video + audio; offsets are 64-row aligned.
    5: Workload(5, "packed_ref_target_audio",
                (_video((8, 16, 16), 0), _video((16, 30, 54), 2048),
                 Segment(DENSE1D, (1, 1, 1024), 27968)),
                24, 128, ((2, 8, 8),) * 24, KEEP_RATIO, with_heat=True),
}


def workload(index: int) -> Workload:
    return WORKLOADS[index]


def segment_positions(seg: Segment) -> torch.Tensor:
    """(t, y, x) of every token of a segment in natural order, float64 [len, 3]."""
    T, H, W = seg.grid
    t = torch.arange(T, dtype=torch.float64).view(T, 1, 1).expand(T, H, W)
    y = torch.arange(H, dtype=torch.float64).view(1, H, 1).expand(T, H, W)
    x = torch.arange(W, dtype=torch.float64).view(1, 1, W).expand(T, H, W)
    return torch.stack([t, y, x], dim=-1).reshape(-1, 3)


def _log_uniform(gen, lo, hi):
    u = float(torch.rand((), generator=gen, dtype=torch.float64))
    return math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))


def _flush_round(x: torch.Tensor) -> torch.Tensor:
    x = torch.where(x.abs() < FLUSH_BELOW, torch.zeros_like(x), x)
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, seed: Optional[int] = None, bias_seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Seeded host tensors for one workload.

    Returns q, k, v: bf16 [N, H, D] (token-major, as a fused QKV projection
    emits them) and w_q, w_k: fp32 [H, D, 3D] predictor projection weights
    (columns ordered mean | max | min), std 0.02.
    Draw order: Q, K, V noise; per-head bias parameters; W_q; W_k.
    bias_seed: draw the per-head bias parameters from their own generator
    with this seed instead (several samples of one layer: the heads keep their
    length scales while the noise changes).
    """
    seed = w.index if seed is None else seed
    gen = torch.Generator("cpu").manual_seed(seed)
    bgen = gen if bias_seed is None else torch.Generator("cpu").manual_seed(bias_seed)
    N, H, D = w.num_tokens, w.num_heads, w.head_dim
    q = torch.randn((N, H, D), generator=gen, dtype=torch.float32)
    k = torch.randn((N, H, D), generator=gen, dtype=torch.float32)
    v = torch.randn((N, H, D), generator=gen, dtype=torch.float32)
    if w.locality_bias:
        F = D // 2
        amp = math.sqrt(3.0 * math.sqrt(D) / F)
        for h in range(H):
            lt = _log_uniform(bgen, 1.0, 4.0)
            ls = _log_uniform(bgen, 2.0, 8.0)
            g = torch.randn((F, 3), generator=bgen, dtype=torch.float64)
            omega = g / torch.tensor([lt, ls, ls], dtype=torch.float64)
            for seg in w.segments:
                if seg.kind != VIDEO3D:
                    continue   # audio tokens carry no 3-D position
                ang = segment_positions(seg) @ omega.T          # [len, F]
                b = torch.empty((seg.length, D), dtype=torch.float64)
                b[:, 0::2] = amp * torch.cos(ang)
                b[:, 1::2] = amp * torch.sin(ang)
                b32 = b.to(torch.float32)
                sl = slice(seg.offset, seg.offset + seg.length)
                q[sl, h, :] += b32
                k[sl, h, :] += b32
    w_q = torch.randn((H, D, 3 * D), generator=gen, dtype=torch.float32) * 0.02
    w_k = torch.randn((H, D, 3 * D), generator=gen, dtype=torch.float32) * 0.02
    return {"q": _flush_round(q), "k": _flush_round(k), "v": _flush_round(v),
            "w_q": w_q.contiguous(), "w_k": w_k.contiguous()}


def sha256_of(t: torch.Tensor) -> str:
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()


def rotation_seeds(w: Workload, count: int = 4) -> List[int]:
    """Seeds of the rotating input sets that give a new block pattern per call."""
    return [w.index + 100 * m for m in range(count)]
