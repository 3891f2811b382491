"""Thin ctypes binding of libveda (include/veda.h), same names as the C ABI.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Torch tensors provide device memory and the current stream; sizes
and dtypes are checked against the plan before a pointer crosses the ABI, so a
wrong tensor raises here instead of reaching a kernel.  There is no fallback:
if libveda.so is missing or the device is not gfx950, calls raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# Only the in-tree build is ever loaded (no override): tests, smoke and bench
# run exactly the library built from this source tree.
LIB_PATH = os.path.join(_PKG, "libveda.so")

VEDA_OK = 0
VEDA_SEG_VIDEO3D = 0
VEDA_SEG_DENSE1D = 1
VEDA_BUDGET_KEEP_RATIO = 0
VEDA_BUDGET_FIXED_K = 1
VEDA_BUDGET_ALL = 2
VEDA_PERMUTE_FORWARD = 0
VEDA_PERMUTE_INVERSE = 1
VEDA_PERMUTE_FORWARD_TRANSPOSED = 2
VEDA_LAYOUT_PERMUTED = 0
VEDA_LAYOUT_NATURAL = 1

STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "SHAPE", 3: "UNSUPPORTED", 4: "WORKSPACE",
                5: "LAUNCH", 6: "STATE"}


class VedaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("veda %s (%d): %s" % (STATUS_NAMES.get(status, "?"), status, message))
        self.status = status


class Segment(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("t", ctypes.c_int32), ("h", ctypes.c_int32),
                ("w", ctypes.c_int32), ("token_offset", ctypes.c_int64)]


class PlanDesc(ctypes.Structure):
    _fields_ = [("num_segments", ctypes.c_int32), ("segments", ctypes.POINTER(Segment)),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("tile_shape", ctypes.POINTER(ctypes.c_int32)), ("budget_mode", ctypes.c_int32),
                ("keep_num", ctypes.c_int32), ("keep_den", ctypes.c_int32), ("fixed_k", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_segments", ctypes.c_int32),
                ("num_shapes", ctypes.c_int32), ("total_rows", ctypes.c_int64),
                ("total_tiles", ctypes.c_int64), ("total_pairs", ctypes.c_int64),
                ("nnz", ctypes.c_int64), ("max_row_blocks", ctypes.c_int64),
                ("device_table_bytes", ctypes.c_int64), ("score_workspace_bytes", ctypes.c_int64),
                ("transpose_workspace_bytes", ctypes.c_int64), ("bwd_workspace_bytes", ctypes.c_int64),
                ("max_tiles_per_head", ctypes.c_int32), ("uploaded", ctypes.c_int32),
                ("heat_workspace_bytes", ctypes.c_int64), ("reduce_workspace_bytes", ctypes.c_int64)]


# name -> (restype, argtypes)
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGS = {
    "veda_abi_version": (ctypes.c_int, []),
    "veda_available": (_I32, [ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t]),
    "veda_last_error": (ctypes.c_char_p, []),
    "veda_plan_create": (_I32, [ctypes.POINTER(PlanDesc), ctypes.POINTER(_P)]),
    "veda_plan_destroy": (None, [_P]),
    "veda_plan_query": (_I32, [_P, ctypes.POINTER(PlanInfo)]),
    "veda_plan_head": (_I32, [_P, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I64),
                              ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "veda_plan_copy_perm": (_I32, [_P, _I32, _P, _I64]),
    "veda_plan_copy_valid": (_I32, [_P, _I32, _P, _I64]),
    "veda_plan_copy_budgets": (_I32, [_P, _I32, _P, _I64]),
    "veda_plan_copy_row_ptr": (_I32, [_P, _P, _I64]),
    "veda_plan_upload": (_I32, [_P, _P, ctypes.c_size_t, _P]),
    "veda_permute_tiles": (_I32, [_P, _P, _P, _I32, _P]),
    "veda_score_tiles": (_I32, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "veda_permute_qkv": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "veda_score_pooled": (_I32, [_P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "veda_select_blocks": (_I32, [_P, _P, _P, _P, _P, _P]),
    "veda_block_sparse_attn_fwd": (_I32, [_P, _P, _I32, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _P, _P, _P]),
    "veda_block_heat": (_I32, [_P, _P, _P, _P, ctypes.c_float, _P, _P]),
    "veda_dense_lse_heat": (_I32, [_P, _P, _I32, _P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "veda_attn_fwd_lse_heat": (_I32, [_P, _P, _P, _I32, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _I32, _P, _P,
                                      _P, _P, ctypes.c_size_t, _P]),
    "veda_mask_mass": (_I32, [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "veda_output_error": (_I32, [_P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "veda_mask_transpose": (_I32, [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "veda_block_sparse_attn_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                          _P, ctypes.c_size_t, _P]),
    "veda_tile_plan_vote": (_I32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_int32, _P]),
    "veda_score_tiles_noalloc": (_I32, [_P, _P, _P, _P, _P, _P, _P]),
}
EXPORTED = tuple(_SIGS)
ABI_VERSION = 9   # the signatures above; a library built from other sources is refused

_lib = None


def lib() -> ctypes.CDLL:
    """Load libveda.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libveda.so is not built (%s); run "
                              "python -m block_sparse_attention_10_amd.build" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        if l.veda_abi_version() != ABI_VERSION:
            raise ImportError("%s has ABI version %d, this binding needs %d; rebuild it with "
                              "python -m block_sparse_attention_10_amd.build" % (LIB_PATH, l.veda_abi_version(),
                                                                                 ABI_VERSION))
        _lib = l
    return _lib


def loaded_library() -> str:
    """Absolute path of the libveda.so this process loaded (loads it)."""
    return os.path.realpath(lib()._name)


def _check(status: int) -> None:
    if status != VEDA_OK:
        raise VedaError(status, lib().veda_last_error().decode())


# ---------------------------------------------------------------------------
# direct wrappers (same names as the C ABI)
# ---------------------------------------------------------------------------

def veda_abi_version() -> int:
    return lib().veda_abi_version()


def veda_available(device: int = 0) -> Tuple[bool, str]:
    buf = ctypes.create_string_buffer(256)
    st = lib().veda_available(device, buf, 256)
    return st == VEDA_OK, buf.value.decode()


def veda_last_error() -> str:
    return lib().veda_last_error().decode()


def veda_plan_create(segments: Sequence, num_heads: int, head_dim: int,
                     tile_shapes: Sequence[Tuple[int, int, int]], budget_mode: int,
                     keep_num: int = 1, keep_den: int = 10, fixed_k: int = 0) -> int:
    """segments: objects with .kind, .grid (t, h, w) and .offset, or tuples
    (kind, (t, h, w), offset).  Returns the plan handle."""
    segs = (Segment * len(segments))()
    for i, s in enumerate(segments):
        kind, grid, off = (s.kind, s.grid, s.offset) if hasattr(s, "kind") else s
        segs[i] = Segment(kind, grid[0], grid[1], grid[2], off)
    shapes = (ctypes.c_int32 * (3 * len(tile_shapes)))(*[x for t in tile_shapes for x in t])
    desc = PlanDesc(len(segments), segs, num_heads, head_dim, shapes, budget_mode,
                    keep_num, keep_den, fixed_k)
    out = _P()
    _check(lib().veda_plan_create(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def veda_plan_destroy(plan: int) -> None:
    lib().veda_plan_destroy(plan)


def veda_plan_query(plan: int) -> Dict[str, int]:
    info = PlanInfo()
    _check(lib().veda_plan_query(plan, ctypes.byref(info)))
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def veda_plan_head(plan: int, head: int) -> Tuple[int, int, int, int]:
    n, r, t, p = _I32(), _I64(), _I64(), _I64()
    _check(lib().veda_plan_head(plan, head, ctypes.byref(n), ctypes.byref(r), ctypes.byref(t),
                                ctypes.byref(p)))
    return n.value, r.value, t.value, p.value


def _copy(fn, plan, n, *head):
    out = np.zeros(n, dtype=np.int32)
    _check(fn(plan, *head, out.ctypes.data, n))
    return out


def veda_plan_copy_perm(plan: int, head: int) -> np.ndarray:
    n = veda_plan_head(plan, head)[0]
    return _copy(lib().veda_plan_copy_perm, plan, 128 * n, head)


def veda_plan_copy_valid(plan: int, head: int) -> np.ndarray:
    n = veda_plan_head(plan, head)[0]
    return _copy(lib().veda_plan_copy_valid, plan, n, head)


def veda_plan_copy_budgets(plan: int, head: int) -> np.ndarray:
    n = veda_plan_head(plan, head)[0]
    S = veda_plan_query(plan)["num_segments"]
    return _copy(lib().veda_plan_copy_budgets, plan, n * S, head).reshape(n, S)


def veda_plan_copy_row_ptr(plan: int) -> np.ndarray:
    T = veda_plan_query(plan)["total_tiles"]
    out = np.zeros(T + 1, dtype=np.int32)
    _check(lib().veda_plan_copy_row_ptr(plan, out.ctypes.data, T + 1))
    return out


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def veda_plan_upload(plan: int, dev_tables, stream=None) -> None:
    _check(lib().veda_plan_upload(plan, dev_tables.data_ptr(), dev_tables.numel() * dev_tables.element_size(),
                                  _stream(stream)))


def veda_permute_tiles(plan: int, src, dst, direction: int, stream=None) -> None:
    _check(lib().veda_permute_tiles(plan, _ptr(src), _ptr(dst), direction, _stream(stream)))


def veda_score_tiles(plan: int, q_perm, k_perm, w_q, w_k, scores, workspace, stream=None) -> None:
    _check(lib().veda_score_tiles(plan, _ptr(q_perm), _ptr(k_perm), _ptr(w_q), _ptr(w_k), _ptr(scores),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)))


def veda_score_tiles_noalloc(plan: int, q_perm, k_perm, w_q, w_k, scores, stream=None) -> None:
    _check(lib().veda_score_tiles_noalloc(plan, _ptr(q_perm), _ptr(k_perm), _ptr(w_q), _ptr(w_k), _ptr(scores),
                                          _stream(stream)))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def veda_permute_qkv(plan: int, q, k, v, q_perm, k_perm, v_t, workspace=None, stream=None) -> None:
    _check(lib().veda_permute_qkv(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(q_perm), _ptr(k_perm), _ptr(v_t),
                                  _ptr(workspace), _nbytes(workspace), _stream(stream)))


def veda_score_pooled(plan: int, w_q, w_k, scores, workspace, stream=None) -> None:
    _check(lib().veda_score_pooled(plan, _ptr(w_q), _ptr(w_k), _ptr(scores), _ptr(workspace),
                                   _nbytes(workspace), _stream(stream)))


def veda_select_blocks(plan: int, scores, row_ptr, col_idx, dense_mask=None, stream=None) -> None:
    _check(lib().veda_select_blocks(plan, _ptr(scores), _ptr(row_ptr), _ptr(col_idx), _ptr(dense_mask),
                                    _stream(stream)))


def veda_block_sparse_attn_fwd(plan: int, q, k, v_t, row_ptr, col_idx, softmax_scale: float, o,
                               o_layout: int = VEDA_LAYOUT_PERMUTED, lse=None, blocks_visited=None,
                               stream=None, q_layout: int = VEDA_LAYOUT_PERMUTED) -> None:
    _check(lib().veda_block_sparse_attn_fwd(plan, _ptr(q), int(q_layout), _ptr(k), _ptr(v_t), _ptr(row_ptr),
                                            _ptr(col_idx), float(softmax_scale), _ptr(o), int(o_layout), _ptr(lse),
                                            _ptr(blocks_visited), _stream(stream)))


def veda_block_heat(plan: int, q, k, lse, softmax_scale: float, heat, stream=None) -> None:
    _check(lib().veda_block_heat(plan, _ptr(q), _ptr(k), _ptr(lse), float(softmax_scale), _ptr(heat),
                                 _stream(stream)))


def veda_dense_lse_heat(plan: int, q, k, row_ptr, col_idx, softmax_scale: float, lse, heat, workspace,
                        stream=None, q_layout: int = VEDA_LAYOUT_PERMUTED) -> None:
    _check(lib().veda_dense_lse_heat(plan, _ptr(q), int(q_layout), _ptr(k), _ptr(row_ptr), _ptr(col_idx),
                                     float(softmax_scale), _ptr(lse), _ptr(heat), _ptr(workspace),
                                     _nbytes(workspace), _stream(stream)))


def veda_attn_fwd_lse_heat(plan: int, dense_plan: int, q, k, v_t, row_ptr, col_idx, dense_row_ptr, dense_col_idx,
                           softmax_scale: float, o, lse, dense_lse, heat, workspace, stream=None,
                           o_layout: int = VEDA_LAYOUT_PERMUTED, q_layout: int = VEDA_LAYOUT_PERMUTED) -> None:
    _check(lib().veda_attn_fwd_lse_heat(plan, dense_plan, _ptr(q), int(q_layout), _ptr(k), _ptr(v_t), _ptr(row_ptr),
                                        _ptr(col_idx), _ptr(dense_row_ptr), _ptr(dense_col_idx),
                                        float(softmax_scale), _ptr(o), int(o_layout), _ptr(lse), _ptr(dense_lse),
                                        _ptr(heat), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def veda_mask_mass(plan: int, heat, row_ptr, col_idx, mass, workspace, stream=None) -> None:
    _check(lib().veda_mask_mass(plan, _ptr(heat), _ptr(row_ptr), _ptr(col_idx), _ptr(mass), _ptr(workspace),
                                _nbytes(workspace), _stream(stream)))


def veda_output_error(plan: int, o, o_ref, err, workspace, stream=None) -> None:
    _check(lib().veda_output_error(plan, _ptr(o), _ptr(o_ref), _ptr(err), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)))


def veda_mask_transpose(plan: int, row_ptr, col_idx, col_ptr, row_idx, workspace, stream=None) -> None:
    _check(lib().veda_mask_transpose(plan, _ptr(row_ptr), _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx),
                                     _ptr(workspace), _nbytes(workspace), _stream(stream)))


def veda_block_sparse_attn_bwd(plan: int, q, k, v, o, d_o, lse, row_ptr, col_idx, col_ptr, row_idx,
                               softmax_scale: float, dq, dk, dv, workspace, stream=None) -> None:
    _check(lib().veda_block_sparse_attn_bwd(plan, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                                            _ptr(row_ptr), _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx),
                                            float(softmax_scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                            _nbytes(workspace), _stream(stream)))


def veda_tile_plan_vote(err, max_shapes: int = 2):
    """err: host float64 array [samples, candidates, heads]; returns int32
    [heads] candidate indices (host-only step, no device)."""
    import numpy as np
    e = np.ascontiguousarray(err, dtype=np.float64)
    if e.ndim != 3:
        raise ValueError("err must be [samples, candidates, heads]")
    out = np.zeros(e.shape[2], dtype=np.int32)
    _check(lib().veda_tile_plan_vote(e.shape[0], e.shape[1], e.shape[2], e.ctypes.data, int(max_shapes),
                                     out.ctypes.data))
    return out


# ---------------------------------------------------------------------------
# Plan: owns the handle and the device tables; checks tensor sizes
# ---------------------------------------------------------------------------

class Plan:
    """A host plan plus its uploaded device tables on the current GPU."""

    def __init__(self, segments, num_heads, head_dim, tile_shapes, budget_mode,
                 keep_num=1, keep_den=10, fixed_k=0, upload=True):
        self.handle = veda_plan_create(segments, num_heads, head_dim, tile_shapes, budget_mode,
                                       keep_num, keep_den, fixed_k)
        self.info = veda_plan_query(self.handle)
        self.tables = None
        if upload:
            self.upload()

    @classmethod
    def from_workload(cls, w, budget_mode=None, upload=True):
        mode = w.budget_mode if budget_mode is None else budget_mode
        return cls(w.segments, w.num_heads, w.head_dim, w.tile_shapes, mode, w.keep_num, w.keep_den,
                   w.fixed_k, upload=upload)

    def upload(self):
        import torch
        self.tables = torch.empty(self.info["device_table_bytes"], dtype=torch.uint8, device="cuda")
        veda_plan_upload(self.handle, self.tables)
        self.info = veda_plan_query(self.handle)

    def close(self):
        if self.handle:
            veda_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # sizes
    @property
    def N(self):
        return self.info["num_tokens"]

    @property
    def H(self):
        return self.info["num_heads"]

    @property
    def D(self):
        return self.info["head_dim"]

    @property
    def R(self):
        return self.info["total_rows"]

    @property
    def T(self):
        return self.info["total_tiles"]

    def _expect(self, t, shape, dtype, name):
        import torch
        if t is None:
            raise ValueError("%s is None" % name)
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous CUDA tensor" % name)
        if t.dtype != dtype or tuple(t.shape) != tuple(shape):
            raise ValueError("%s: expected %s %s, got %s %s" % (name, dtype, tuple(shape), t.dtype,
                                                               tuple(t.shape)))

    # calls
    def permute(self, src, dst, direction, stream=None):
        import torch
        bf = torch.bfloat16
        nat = (self.N, self.H, self.D)
        if direction == VEDA_PERMUTE_INVERSE:
            self._expect(src, (self.R, self.D), bf, "src")
            self._expect(dst, nat, bf, "dst")
        elif direction == VEDA_PERMUTE_FORWARD:
            self._expect(src, nat, bf, "src")
            self._expect(dst, (self.R, self.D), bf, "dst")
        else:
            self._expect(src, nat, bf, "src")
            self._expect(dst, (self.T, self.D, 128), bf, "dst")
        veda_permute_tiles(self.handle, src, dst, direction, stream)

    def permute_qkv(self, q, k, v, q_perm, k_perm, v_t, workspace=None, stream=None):
        import torch
        bf = torch.bfloat16
        nat = (self.N, self.H, self.D)
        for t, n in ((q, "q"), (k, "k")):
            self._expect(t, nat, bf, n)
        if q_perm is None:      # Q pooled, not written (attention then reads natural Q)
            if workspace is None:
                raise ValueError("permute_qkv: q_perm=None needs the pooling workspace")
        else:
            self._expect(q_perm, (self.R, self.D), bf, "q_perm")
        self._expect(k_perm, (self.R, self.D), bf, "k_perm")
        if (v is None) != (v_t is None):
            raise ValueError("permute_qkv: give both v and v_t, or neither")
        if v is not None:
            self._expect(v, nat, bf, "v")
            self._expect(v_t, (self.T, self.D, 128), bf, "v_t")
        if workspace is not None:
            self._check_workspace(workspace)
        veda_permute_qkv(self.handle, q, k, v, q_perm, k_perm, v_t, workspace, stream)

    def score_pooled(self, w_q, w_k, scores, workspace, stream=None):
        import torch
        self._expect(w_q, (self.H, self.D, 3 * self.D), torch.float32, "w_q")
        self._expect(w_k, (self.H, self.D, 3 * self.D), torch.float32, "w_k")
        self._expect(scores, (self.info["total_pairs"],), torch.float32, "scores")
        self._check_workspace(workspace)
        veda_score_pooled(self.handle, w_q, w_k, scores, workspace, stream)

    def _check_workspace(self, ws):
        if ws is None or not ws.is_cuda or not ws.is_contiguous() or _nbytes(ws) < self.info["score_workspace_bytes"]:
            raise ValueError("workspace must be a contiguous CUDA tensor of >= %d bytes"
                             % self.info["score_workspace_bytes"])

    def score(self, q_perm, k_perm, w_q, w_k, scores, workspace, stream=None):
        import torch
        self._expect(q_perm, (self.R, self.D), torch.bfloat16, "q_perm")
        self._expect(k_perm, (self.R, self.D), torch.bfloat16, "k_perm")
        self._expect(w_q, (self.H, self.D, 3 * self.D), torch.float32, "w_q")
        self._expect(w_k, (self.H, self.D, 3 * self.D), torch.float32, "w_k")
        self._expect(scores, (self.info["total_pairs"],), torch.float32, "scores")
        self._check_workspace(workspace)
        veda_score_tiles(self.handle, q_perm, k_perm, w_q, w_k, scores, workspace, stream)

    def score_noalloc(self, q_perm, k_perm, w_q, w_k, scores, stream=None):
        """veda_score_tiles with the library's static scratch (no workspace)."""
        import torch
        self._expect(q_perm, (self.R, self.D), torch.bfloat16, "q_perm")
        self._expect(k_perm, (self.R, self.D), torch.bfloat16, "k_perm")
        self._expect(w_q, (self.H, self.D, 3 * self.D), torch.float32, "w_q")
        self._expect(w_k, (self.H, self.D, 3 * self.D), torch.float32, "w_k")
        self._expect(scores, (self.info["total_pairs"],), torch.float32, "scores")
        veda_score_tiles_noalloc(self.handle, q_perm, k_perm, w_q, w_k, scores, stream)

    def select(self, scores, row_ptr, col_idx, dense_mask=None, stream=None):
        import torch
        self._expect(scores, (self.info["total_pairs"],), torch.float32, "scores")
        self._expect(row_ptr, (self.T + 1,), torch.int32, "row_ptr")
        self._expect(col_idx, (self.info["nnz"],), torch.int32, "col_idx")
        if dense_mask is not None:
            self._expect(dense_mask, (self.info["total_pairs"],), torch.uint8, "dense_mask")
        veda_select_blocks(self.handle, scores, row_ptr, col_idx, dense_mask, stream)

    def _expect_q(self, q, q_layout):
        import torch
        if q_layout == VEDA_LAYOUT_NATURAL:
            self._expect(q, (self.N, self.H, self.D), torch.bfloat16, "q")
        else:
            self._expect(q, (self.R, self.D), torch.bfloat16, "q")

    def attention(self, q, k, v_t, row_ptr, col_idx, scale, o, lse=None, visited=None, stream=None,
                  o_layout=VEDA_LAYOUT_PERMUTED, q_layout=VEDA_LAYOUT_PERMUTED):
        import torch
        bf = torch.bfloat16
        self._expect_q(q, q_layout)
        self._expect(k, (self.R, self.D), bf, "k")
        self._expect(v_t, (self.T, self.D, 128), bf, "v_t")
        self._expect(row_ptr, (self.T + 1,), torch.int32, "row_ptr")
        if col_idx is None or col_idx.dtype != torch.int32 or not col_idx.is_cuda:
            raise ValueError("col_idx must be an int32 CUDA tensor")
        if o is None:          # only the LSE
            if lse is None:
                raise ValueError("attention: o and lse are both None")
        elif o_layout == VEDA_LAYOUT_NATURAL:
            self._expect(o, (self.N, self.H, self.D), bf, "o")
        else:
            self._expect(o, (self.R, self.D), bf, "o")
        if lse is not None:
            self._expect(lse, (self.R,), torch.float32, "lse")
        if visited is not None:
            self._expect(visited, (1,), torch.int32, "blocks_visited")
        veda_block_sparse_attn_fwd(self.handle, q, k, v_t, row_ptr, col_idx, scale, o, o_layout, lse, visited,
                                   stream, q_layout)

    def heat(self, q, k, lse, scale, heat, stream=None):
        import torch
        self._expect(q, (self.R, self.D), torch.bfloat16, "q")
        self._expect(k, (self.R, self.D), torch.bfloat16, "k")
        self._expect(lse, (self.R,), torch.float32, "lse")
        self._expect(heat, (self.info["total_pairs"],), torch.float32, "heat")
        veda_block_heat(self.handle, q, k, lse, scale, heat, stream)

    def lse_heat(self, q, k, row_ptr, col_idx, scale, lse, heat, workspace, stream=None,
                 q_layout=VEDA_LAYOUT_PERMUTED):
        import torch
        self._expect_q(q, q_layout)
        self._expect(k, (self.R, self.D), torch.bfloat16, "k")
        self._expect(row_ptr, (self.T + 1,), torch.int32, "row_ptr")
        self._expect(col_idx, (self.info["nnz"],), torch.int32, "col_idx")
        if lse is not None:
            self._expect(lse, (self.R,), torch.float32, "lse")
        self._expect(heat, (self.info["total_pairs"],), torch.float32, "heat")
        self._check_ws(workspace, "heat_workspace_bytes")
        veda_dense_lse_heat(self.handle, q, k, row_ptr, col_idx, scale, lse, heat, workspace, stream, q_layout)

    def attention_lse_heat(self, dense, q, k, v_t, row_ptr, col_idx, dense_row_ptr, dense_col_idx, scale, o, lse,
                           dense_lse, heat, workspace, stream=None, o_layout=VEDA_LAYOUT_PERMUTED,
                           q_layout=VEDA_LAYOUT_PERMUTED):
        """attention() over this plan's selected CSR and dense.lse_heat() over
        the dense plan's all-blocks CSR, in one pass (veda_attn_fwd_lse_heat)."""
        import torch
        bf = torch.bfloat16
        self._expect_q(q, q_layout)
        self._expect(k, (self.R, self.D), bf, "k")
        self._expect(v_t, (self.T, self.D, 128), bf, "v_t")
        self._expect(row_ptr, (self.T + 1,), torch.int32, "row_ptr")
        self._expect(col_idx, (self.info["nnz"],), torch.int32, "col_idx")
        self._expect(dense_row_ptr, (dense.T + 1,), torch.int32, "dense_row_ptr")
        self._expect(dense_col_idx, (dense.info["nnz"],), torch.int32, "dense_col_idx")
        if o_layout == VEDA_LAYOUT_NATURAL:
            self._expect(o, (self.N, self.H, self.D), bf, "o")
        else:
            self._expect(o, (self.R, self.D), bf, "o")
        for name, x in (("lse", lse), ("dense_lse", dense_lse)):
            if x is not None:
                self._expect(x, (self.R,), torch.float32, name)
        self._expect(heat, (self.info["total_pairs"],), torch.float32, "heat")
        dense._check_ws(workspace, "heat_workspace_bytes")
        veda_attn_fwd_lse_heat(self.handle, dense.handle, q, k, v_t, row_ptr, col_idx, dense_row_ptr, dense_col_idx,
                               scale, o, lse, dense_lse, heat, workspace, stream, o_layout, q_layout)

    def transpose(self, row_ptr, col_idx, col_ptr, row_idx, workspace, stream=None):
        import torch
        self._expect(row_ptr, (self.T + 1,), torch.int32, "row_ptr")
        self._expect(col_idx, (self.info["nnz"],), torch.int32, "col_idx")
        self._expect(col_ptr, (self.T + 1,), torch.int32, "col_ptr")
        self._expect(row_idx, (self.info["nnz"],), torch.int32, "row_idx")
        self._check_ws(workspace, "transpose_workspace_bytes")
        veda_mask_transpose(self.handle, row_ptr, col_idx, col_ptr, row_idx, workspace, stream)

    def backward(self, q, k, v, o, d_o, lse, row_ptr, col_idx, col_ptr, row_idx, scale, dq, dk, dv, workspace,
                 stream=None):
        import torch
        bf = torch.bfloat16
        for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (d_o, "d_o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
            self._expect(t, (self.R, self.D), bf, name)
        self._expect(lse, (self.R,), torch.float32, "lse")
        self._expect(row_ptr, (self.T + 1,), torch.int32, "row_ptr")
        self._expect(col_idx, (self.info["nnz"],), torch.int32, "col_idx")
        self._expect(col_ptr, (self.T + 1,), torch.int32, "col_ptr")
        self._expect(row_idx, (self.info["nnz"],), torch.int32, "row_idx")
        self._check_ws(workspace, "bwd_workspace_bytes")
        veda_block_sparse_attn_bwd(self.handle, q, k, v, o, d_o, lse, row_ptr, col_idx, col_ptr, row_idx, scale,
                                   dq, dk, dv, workspace, stream)

    def _check_ws(self, ws, key):
        if ws is None or not ws.is_cuda or not ws.is_contiguous() or _nbytes(ws) < self.info[key]:
            raise ValueError("workspace must be a contiguous CUDA tensor of at least %d bytes" % self.info[key])

    def empty_bytes(self, key):
        import torch
        return torch.empty(max(self.info[key], 1), dtype=torch.uint8, device="cuda")

    def _reduce_ws(self, workspace):
        # the two-launch reductions' partial sums: a given buffer, else one
        # torch buffer kept with the plan (calls on one stream reuse it)
        if workspace is not None:
            self._check_ws(workspace, "reduce_workspace_bytes")
            return workspace
        if getattr(self, "_rws", None) is None:
            self._rws = self.empty_bytes("reduce_workspace_bytes")
        return self._rws

    def output_error(self, o, o_ref, err, workspace=None, stream=None):
        import torch
        nat = (self.N, self.H, self.D)
        self._expect(o, nat, torch.bfloat16, "o")
        self._expect(o_ref, nat, torch.bfloat16, "o_ref")
        self._expect(err, (self.H,), torch.float64, "err")
        veda_output_error(self.handle, o, o_ref, err, self._reduce_ws(workspace), stream)

    def mask_mass(self, heat, row_ptr, col_idx, mass, workspace=None, stream=None):
        import torch
        self._expect(heat, (self.info["total_pairs"],), torch.float32, "heat")
        self._expect(row_ptr, (self.T + 1,), torch.int32, "row_ptr")
        if col_idx is None or col_idx.dtype != torch.int32 or not col_idx.is_cuda:
            raise ValueError("col_idx must be a device int32 tensor")
        self._expect(mass, (self.H,), torch.float64, "mass")
        veda_mask_mass(self.handle, heat, row_ptr, col_idx, mass, self._reduce_ws(workspace), stream)

    # allocation helpers (torch: device memory only)
    def empty_perm(self):
        import torch
        return torch.empty((self.R, self.D), dtype=torch.bfloat16, device="cuda")

    def empty_vt(self):
        import torch
        return torch.empty((self.T, self.D, 128), dtype=torch.bfloat16, device="cuda")

    def empty_workspace(self):
        import torch
        return torch.empty(self.info["score_workspace_bytes"] // 4, dtype=torch.float32, device="cuda")

    def score_workspace_views(self, workspace):
        """Named views of a score workspace (fp32 tensor of score_workspace_bytes)
        in the layout include/veda.h documents for veda_score_tiles: pooled
        features of Q and K [T, 3D], then the projections q_hat, k_hat [T, D]."""
        self._check_workspace(workspace)
        T, D = self.T, self.D
        w = workspace.view(-1)
        f = T * 3 * D
        return {"feat_q": w[0:f].view(T, 3 * D), "feat_k": w[f:2 * f].view(T, 3 * D),
                "q_hat": w[2 * f:2 * f + T * D].view(T, D), "k_hat": w[2 * f + T * D:2 * f + 2 * T * D].view(T, D)}
