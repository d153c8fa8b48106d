"""Thin ctypes binding of libjssa.so (include/jssa.h): argument marshalling only.

Every function takes torch tensors, checks dtype / device / contiguity / size
against the shape on the host (the C ABI sees plain pointers and cannot), and
passes data pointers plus the current HIP stream.  All arithmetic happens in
the library's HIP kernels; there is no fallback: if libjssa.so is missing the
import fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libjssa.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN = 0, -1, -2, -3, -4, -5, -6
KIND_GQA, KIND_MLA = 0, 1
SELECT_AUTO, SELECT_EXACT_STREAM, SELECT_SPLIT, SELECT_FUSED = 0, 1, 2, 3
SCALE_FP32, SCALE_E8M0, SCALE_NONE, KEYS_BF16 = 0, 1, 2, 3
SCALE_FORMATS = {"fp32": SCALE_FP32, "e8m0": SCALE_E8M0, "none": SCALE_NONE, "bf16": KEYS_BF16}
STAGE_PROLOGUE, STAGE_STREAM, STAGE_FINISH, STAGE_ALL = 1, 2, 4, 7
MLA_LATENT, MLA_ROPE = 512, 64

EXPORTED = ("jssa_status_string", "jssa_workspace_bytes", "jssa_decode_path", "jssa_attend_splits",
            "jssa_kp_page_bytes", "jssa_store",
            "jssa_select",
            "jssa_select_stages",
            "jssa_attend", "jssa_attend_noalloc", "jssa_decode", "jssa_full_decode", "jssa_gather_attend", "jssa_calib_workspace_bytes",
            "jssa_calib_moments", "jssa_basis")


class JSSAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "kind", "batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "max_pages_per_seq",
        "rank", "budget", "select_mode", "scale_format")]

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def score_dims(self) -> int:
        return self.rank + (MLA_ROPE if self.kind == KIND_MLA else 0)

    @property
    def v_dim(self) -> int:
        return MLA_LATENT if self.kind == KIND_MLA else self.head_dim


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    S = ctypes.POINTER(Shape)
    sig = {
        "jssa_status_string": (ctypes.c_char_p, [I32]),
        "jssa_workspace_bytes": (I32, [S, ctypes.POINTER(SZ)]),
        "jssa_decode_path": (I32, [S, ctypes.POINTER(I32)]),
        "jssa_attend_splits": (I32, [S, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "jssa_kp_page_bytes": (I32, [S, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
        "jssa_store": (I32, [S, P, P, I32, P, P, P, P]),
        "jssa_select": (I32, [S, P, P, P, P, P, P, P, P, P, SZ, P]),
        "jssa_select_stages": (I32, [S, I32, P, P, P, P, P, P, P, P, P, SZ, P]),
        "jssa_attend": (I32, [S, P, P, P, P, P, P, ctypes.c_float, P, P, P, SZ, P]),
        "jssa_attend_noalloc": (I32, [S, P, P, P, P, P, P, ctypes.c_float, P, P, P]),
        "jssa_decode": (I32, [S, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, SZ, P]),
        "jssa_full_decode": (I32, [S, P, P, P, P, P, I32, ctypes.c_float, P, P, P, SZ, P]),
        "jssa_gather_attend": (I32, [S, P, P, P, P, P, P, ctypes.c_float, P, P, P, SZ, P]),
        "jssa_calib_workspace_bytes": (I32, [S, I32, ctypes.POINTER(SZ)]),
        "jssa_calib_moments": (I32, [S, P, P, I32, P, P, P, SZ, P]),
        "jssa_basis": (I32, [S, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.jssa_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise JSSAError(fn, status)


def make_shape(kind: int, batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
               max_pages_per_seq: int, rank: int, budget: int, select_mode: int = SELECT_AUTO,
               scale_format: int = SCALE_FP32) -> Shape:
    return Shape(kind, batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq, rank, budget,
                 select_mode, scale_format)


def shape_for(w, select_mode: int = SELECT_AUTO, batch: Optional[int] = None,
              max_pages_per_seq: Optional[int] = None, scale_format: int = SCALE_FP32) -> Shape:
    """Shape of a synth Workload (duck-typed: any object with the same fields)."""
    return make_shape(KIND_MLA if w.kind == "mla" else KIND_GQA, batch or w.batch, w.num_q_heads, w.num_kv_heads,
                      w.head_dim, w.page_size, max_pages_per_seq or w.pages_per_seq, w.rank, w.budget, select_mode,
                      scale_format)


def workspace_bytes(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check("jssa_workspace_bytes", _lib.jssa_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def decode_single_launch(shape: Shape) -> bool:
    """Whether jssa_decode runs this shape as one launch per layer."""
    v = ctypes.c_int32()
    _check("jssa_decode_path", _lib.jssa_decode_path(ctypes.byref(shape), ctypes.byref(v)))
    return bool(v.value)


def attend_splits(shape: Shape, sparse: bool, window: int = 0) -> Tuple[int, int]:
    """(splits an attention call of this shape uses, splits the workspace holds)."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check("jssa_attend_splits", _lib.jssa_attend_splits(ctypes.byref(shape), int(bool(sparse)), int(window),
                                                         ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def kp_page_bytes(shape: Shape) -> Tuple[int, int]:
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check("jssa_kp_page_bytes", _lib.jssa_kp_page_bytes(ctypes.byref(shape), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


# ---------------------------------------------------------------- allocation helpers

def alloc_workspace(shape: Shape, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_bytes(shape), dtype=torch.uint8, device=device)


def _scale_dtype(shape: Shape):
    return {SCALE_FP32: torch.float32, SCALE_E8M0: torch.uint8}.get(shape.scale_format)


def _kp_pieces(shape: Shape) -> int:
    """16-byte pieces per (token, KV head): S/16 FP8 codes, 2S/16 for BF16 keys."""
    return shape.score_dims // 16 * (2 if shape.scale_format == KEYS_BF16 else 1)


def alloc_scoring_cache(shape: Shape, num_pages: int, device="cuda") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Zeroed projected scoring cache: kp uint8 [num_pages, Hkv, S/16, page, 16] (BF16 keys: 2S/16
    pieces) and the scales [num_pages, Hkv, page] (fp32, or uint8 E8M0 bytes; None when the format has
    no scale)."""
    kp = torch.zeros((num_pages, shape.num_kv_heads, _kp_pieces(shape), shape.page_size, 16), dtype=torch.uint8,
                     device=device)
    dt = _scale_dtype(shape)
    sc = None if dt is None else torch.zeros((num_pages, shape.num_kv_heads, shape.page_size), dtype=dt, device=device)
    return kp, sc


# ---------------------------------------------------------------- argument checks

def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(name: str, t: Optional[torch.Tensor], dtype, shape=None, optional=False) -> ctypes.c_void_p:
    if t is None:
        if optional:
            return ctypes.c_void_p(0)
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _cache_shape(shape: Shape, cache: torch.Tensor):
    """(num_pages, expected cache shape) of a paged K/V or latent cache."""
    n = cache.shape[0]
    if shape.kind == KIND_MLA:
        return n, (n, shape.page_size, shape.head_dim)
    return n, (n, shape.page_size, shape.num_kv_heads, shape.head_dim)


def _m_shape(shape: Shape):
    if shape.kind == KIND_MLA:
        return (shape.rank, MLA_LATENT)
    return (shape.num_kv_heads, shape.rank, shape.head_dim)


def _kp_args(shape: Shape, kp: torch.Tensor, kp_scale: Optional[torch.Tensor]):
    n = kp.shape[0]
    dt = _scale_dtype(shape)
    if dt is None:
        if kp_scale is not None:
            raise ValueError("kp_scale: this scale format stores no scale (pass None)")
        sc = ctypes.c_void_p(0)
    else:
        sc = _ptr("kp_scale", kp_scale, dt, (n, shape.num_kv_heads, shape.page_size))
    return (_ptr("kp", kp, torch.uint8, (n, shape.num_kv_heads, _kp_pieces(shape), shape.page_size, 16)), sc)


def _ws(shape: Shape, workspace: torch.Tensor):
    need = workspace_bytes(shape)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or workspace.numel() < need:
        raise ValueError(f"workspace: need a device uint8 tensor of >= {need} bytes")
    return ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel())


def _table_args(shape: Shape, block_table: torch.Tensor, seq_lens: torch.Tensor):
    return (_ptr("block_table", block_table, torch.int32, (shape.batch, shape.max_pages_per_seq)),
            _ptr("seq_lens", seq_lens, torch.int32, (shape.batch,)))


# ---------------------------------------------------------------- entry points

def jssa_store(shape: Shape, k_new: torch.Tensor, slot: torch.Tensor, M: torch.Tensor, kp: torch.Tensor,
               kp_scale: Optional[torch.Tensor], check_slots: bool = True) -> None:
    """check_slots=True reads the slots back to the host (a synchronisation) to bound-check them."""
    T = int(slot.shape[0])
    kshape = (T, shape.head_dim) if shape.kind == KIND_MLA else (T, shape.num_kv_heads, shape.head_dim)
    args = (_ptr("k_new", k_new, torch.bfloat16, kshape),
            _ptr("slot", slot, torch.int32, (T,)), ctypes.c_int32(T), _ptr("M", M, torch.float32, _m_shape(shape)),
            *_kp_args(shape, kp, kp_scale))
    if T and check_slots:
        if int(slot.max().item()) >= kp.shape[0] * shape.page_size:
            raise ValueError("slot beyond the scoring cache")
    _check("jssa_store", _lib.jssa_store(ctypes.byref(shape), *args, _stream()))


def jssa_select(shape: Shape, q: torch.Tensor, M: torch.Tensor, kp: torch.Tensor, kp_scale: Optional[torch.Tensor],
                block_table: torch.Tensor, seq_lens: torch.Tensor, indices: torch.Tensor,
                workspace: torch.Tensor, scores_out: Optional[torch.Tensor] = None,
                stages: Optional[int] = None) -> None:
    """stages=None calls jssa_select; a STAGE_* mask calls jssa_select_stages."""
    maxn = shape.max_pages_per_seq * shape.page_size
    args = (_ptr("q", q, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.head_dim)),
            _ptr("M", M, torch.float32, _m_shape(shape)), *_kp_args(shape, kp, kp_scale),
            *_table_args(shape, block_table, seq_lens),
            _ptr("indices", indices, torch.int32, (shape.batch, shape.num_kv_heads, shape.budget)),
            _ptr("scores_out", scores_out, torch.float32, (shape.batch, shape.num_kv_heads, maxn), optional=True),
            *_ws(shape, workspace))
    if stages is None:
        _check("jssa_select", _lib.jssa_select(ctypes.byref(shape), *args, _stream()))
    else:
        _check("jssa_select_stages", _lib.jssa_select_stages(ctypes.byref(shape), int(stages), *args, _stream()))


def jssa_attend(shape: Shape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                block_table: torch.Tensor, seq_lens: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                out: torch.Tensor, workspace: torch.Tensor, lse_out: Optional[torch.Tensor] = None) -> None:
    n, cs = _cache_shape(shape, k_cache)
    args = (_ptr("q", q, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.head_dim)),
            _ptr("k_cache", k_cache, torch.bfloat16, cs),
            _ptr("v_cache", v_cache, torch.bfloat16, cs, optional=shape.kind == KIND_MLA),
            *_table_args(shape, block_table, seq_lens),
            _ptr("indices", indices, torch.int32, (shape.batch, shape.num_kv_heads, shape.budget)),
            ctypes.c_float(sm_scale),
            _ptr("out", out, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.v_dim)),
            _ptr("lse_out", lse_out, torch.float32, (shape.batch, shape.num_q_heads), optional=True),
            *_ws(shape, workspace))
    _check("jssa_attend", _lib.jssa_attend(ctypes.byref(shape), *args, _stream()))


def jssa_attend_noalloc(shape: Shape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                        block_table: torch.Tensor, seq_lens: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                        out: torch.Tensor, lse_out: Optional[torch.Tensor] = None) -> None:
    """jssa_attend without a workspace (the library's own per-GPU scratch array holds the partials)."""
    n, cs = _cache_shape(shape, k_cache)
    args = (_ptr("q", q, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.head_dim)),
            _ptr("k_cache", k_cache, torch.bfloat16, cs),
            _ptr("v_cache", v_cache, torch.bfloat16, cs, optional=shape.kind == KIND_MLA),
            *_table_args(shape, block_table, seq_lens),
            _ptr("indices", indices, torch.int32, (shape.batch, shape.num_kv_heads, shape.budget)),
            ctypes.c_float(sm_scale),
            _ptr("out", out, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.v_dim)),
            _ptr("lse_out", lse_out, torch.float32, (shape.batch, shape.num_q_heads), optional=True))
    _check("jssa_attend_noalloc", _lib.jssa_attend_noalloc(ctypes.byref(shape), *args, _stream()))


def jssa_decode(shape: Shape, q: torch.Tensor, k_new: Optional[torch.Tensor], slot_new: Optional[torch.Tensor],
                M: torch.Tensor, kp: torch.Tensor, kp_scale: Optional[torch.Tensor], k_cache: torch.Tensor,
                v_cache: Optional[torch.Tensor], block_table: torch.Tensor, seq_lens: torch.Tensor,
                indices: torch.Tensor, sm_scale: float, out: torch.Tensor, workspace: torch.Tensor,
                lse_out: Optional[torch.Tensor] = None) -> None:
    n, cs = _cache_shape(shape, k_cache)
    b = shape.batch
    kshape = (b, shape.head_dim) if shape.kind == KIND_MLA else (b, shape.num_kv_heads, shape.head_dim)
    args = (_ptr("q", q, torch.bfloat16, (b, shape.num_q_heads, shape.head_dim)),
            _ptr("k_new", k_new, torch.bfloat16, kshape, optional=True),
            _ptr("slot_new", slot_new, torch.int32, (b,), optional=k_new is None),
            _ptr("M", M, torch.float32, _m_shape(shape)), *_kp_args(shape, kp, kp_scale),
            _ptr("k_cache", k_cache, torch.bfloat16, cs),
            _ptr("v_cache", v_cache, torch.bfloat16, cs, optional=shape.kind == KIND_MLA),
            *_table_args(shape, block_table, seq_lens),
            _ptr("indices", indices, torch.int32, (b, shape.num_kv_heads, shape.budget)),
            ctypes.c_float(sm_scale),
            _ptr("out", out, torch.bfloat16, (b, shape.num_q_heads, shape.v_dim)),
            _ptr("lse_out", lse_out, torch.float32, (b, shape.num_q_heads), optional=True),
            *_ws(shape, workspace))
    _check("jssa_decode", _lib.jssa_decode(ctypes.byref(shape), *args, _stream()))


def jssa_full_decode(shape: Shape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                     block_table: torch.Tensor, seq_lens: torch.Tensor, window: int, sm_scale: float,
                     out: torch.Tensor, workspace: torch.Tensor, lse_out: Optional[torch.Tensor] = None) -> None:
    n, cs = _cache_shape(shape, k_cache)
    args = (_ptr("q", q, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.head_dim)),
            _ptr("k_cache", k_cache, torch.bfloat16, cs),
            _ptr("v_cache", v_cache, torch.bfloat16, cs, optional=shape.kind == KIND_MLA),
            *_table_args(shape, block_table, seq_lens), ctypes.c_int32(window), ctypes.c_float(sm_scale),
            _ptr("out", out, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.v_dim)),
            _ptr("lse_out", lse_out, torch.float32, (shape.batch, shape.num_q_heads), optional=True),
            *_ws(shape, workspace))
    _check("jssa_full_decode", _lib.jssa_full_decode(ctypes.byref(shape), *args, _stream()))


def jssa_gather_attend(shape: Shape, q: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor],
                       block_table: torch.Tensor, seq_lens: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                       out: torch.Tensor, workspace: torch.Tensor, lse_out: Optional[torch.Tensor] = None) -> None:
    n, cs = _cache_shape(shape, k_cache)
    args = (_ptr("q", q, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.head_dim)),
            _ptr("k_cache", k_cache, torch.bfloat16, cs),
            _ptr("v_cache", v_cache, torch.bfloat16, cs, optional=shape.kind == KIND_MLA),
            *_table_args(shape, block_table, seq_lens),
            _ptr("indices", indices, torch.int32, (shape.batch, shape.num_kv_heads, shape.budget)),
            ctypes.c_float(sm_scale),
            _ptr("out", out, torch.bfloat16, (shape.batch, shape.num_q_heads, shape.v_dim)),
            _ptr("lse_out", lse_out, torch.float32, (shape.batch, shape.num_q_heads), optional=True),
            *_ws(shape, workspace))
    _check("jssa_gather_attend", _lib.jssa_gather_attend(ctypes.byref(shape), *args, _stream()))


def calib_workspace_bytes(shape: Shape, T: int) -> int:
    n = ctypes.c_size_t()
    _check("jssa_calib_workspace_bytes", _lib.jssa_calib_workspace_bytes(ctypes.byref(shape), T, ctypes.byref(n)))
    return n.value


def jssa_calib_moments(shape: Shape, q_cal: torch.Tensor, k_cal: torch.Tensor, gq: torch.Tensor, gk: torch.Tensor,
                       workspace: torch.Tensor) -> None:
    T = int(q_cal.shape[0])
    dm = MLA_LATENT if shape.kind == KIND_MLA else shape.head_dim
    kshape = (T, shape.head_dim) if shape.kind == KIND_MLA else (T, shape.num_kv_heads, shape.head_dim)
    need = calib_workspace_bytes(shape, T)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or workspace.numel() < need:
        raise ValueError(f"workspace: need a device uint8 tensor of >= {need} bytes")
    args = (_ptr("q_cal", q_cal, torch.bfloat16, (T, shape.num_q_heads, shape.head_dim)),
            _ptr("k_cal", k_cal, torch.bfloat16, kshape), ctypes.c_int32(T),
            _ptr("gq", gq, torch.float32, (shape.num_kv_heads, dm, dm)),
            _ptr("gk", gk, torch.float32, (shape.num_kv_heads, dm, dm)),
            ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()))
    _check("jssa_calib_moments", _lib.jssa_calib_moments(ctypes.byref(shape), *args, _stream()))


def jssa_basis(shape: Shape, gq: np.ndarray, gk: np.ndarray) -> np.ndarray:
    """Host eigensolver: fp32 moment sums [Hkv, dm, dm] (numpy) -> M [Hkv, r, dm] (numpy fp32)."""
    dm = MLA_LATENT if shape.kind == KIND_MLA else shape.head_dim
    gq = np.ascontiguousarray(gq, dtype=np.float32)
    gk = np.ascontiguousarray(gk, dtype=np.float32)
    if gq.shape != (shape.num_kv_heads, dm, dm) or gk.shape != gq.shape:
        raise ValueError(f"moments must be [{shape.num_kv_heads}, {dm}, {dm}]")
    m = np.zeros((shape.num_kv_heads, shape.rank, dm), dtype=np.float32)
    _check("jssa_basis", _lib.jssa_basis(ctypes.byref(shape), gq.ctypes.data, gk.ctypes.data, m.ctypes.data))
    return m


def raw_library() -> ctypes.CDLL:
    return _lib
