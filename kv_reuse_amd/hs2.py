"""Thin ctypes binding of libhs2.so (include/hs2.h), with the same entry-point names.

Only argument marshalling happens here: shapes and dtypes are checked, torch
tensors are passed as device pointers, and torch's current HIP stream is
passed as the stream.  Every step of the computation runs in the library's
HIP kernels.  If the library has not been built, importing this module fails.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# HS2_LIBRARY may name another build of the same library (the host-sanitizer
# build of kv_reuse_amd.build --asan-host, for instance)
LIB_PATH = os.environ.get("HS2_LIBRARY") or os.path.join(_HERE, "libhs2.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first (python -m kv_reuse_amd.build "
                      "or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

HS2_OK, HS2_ERR_INVALID_ARG, HS2_ERR_UNSUPPORTED, HS2_ERR_WORKSPACE, HS2_ERR_HIP = 0, -1, -2, -3, -4
HS2_ERR_SCRATCH = -5
HS2_STATIC_SCRATCH_BYTES = 96 << 20   # the library-held buffer of cross_decoder_step_static
EXPORTED = ["hs2_workspace_bytes", "hs2_full_attn_scores", "hs2_topk_select", "hs2_sparse_attn",
            "hs2_cross_decoder_step", "hs2_cross_decoder_step_timed", "hs2_kv_bridge",
            "hs2_sparse_attn_swa", "hs2_workspace_region", "hs2_stream_read_ms",
            "hs2_status_string", "hs2_last_hip_error", "hs2_cross_decoder_step_static"]


class Shape(ctypes.Structure):
    _fields_ = [("ctx_len", ctypes.c_int64), ("scale", ctypes.c_double),
                ("batch", ctypes.c_int32), ("n_q_tokens", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("window", ctypes.c_int32), ("select_block", ctypes.c_int32),
                ("kv_capacity", ctypes.c_int64), ("decode_splits", ctypes.c_int32),
                ("decode_select", ctypes.c_int32)]


class BridgeShape(ctypes.Structure):
    _fields_ = [("kv_capacity", ctypes.c_int64), ("pos0", ctypes.c_int64),
                ("batch", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_SP = ctypes.POINTER(Shape)
_lib.hs2_workspace_bytes.argtypes = [_SP, ctypes.c_int32]
_lib.hs2_workspace_bytes.restype = ctypes.c_size_t
_lib.hs2_full_attn_scores.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.hs2_full_attn_scores.restype = ctypes.c_int
_lib.hs2_topk_select.argtypes = [_SP, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.hs2_topk_select.restype = ctypes.c_int
_lib.hs2_sparse_attn.argtypes = [_SP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
_lib.hs2_sparse_attn.restype = ctypes.c_int
_lib.hs2_cross_decoder_step.argtypes = [_SP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, ctypes.c_size_t, _P]
_lib.hs2_cross_decoder_step.restype = ctypes.c_int
_lib.hs2_cross_decoder_step_timed.argtypes = [_SP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P,
                                              _P, _P, ctypes.c_size_t, _P, ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_float)]
_lib.hs2_cross_decoder_step_timed.restype = ctypes.c_int
_lib.hs2_sparse_attn_swa.argtypes = [_SP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]
_lib.hs2_sparse_attn_swa.restype = ctypes.c_int
_lib.hs2_kv_bridge.argtypes = [ctypes.POINTER(BridgeShape), _P, _P, _P, _P, _P]
_lib.hs2_kv_bridge.restype = ctypes.c_int
_lib.hs2_workspace_region.argtypes = [_SP, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_size_t),
                                      ctypes.POINTER(ctypes.c_size_t)]
_lib.hs2_workspace_region.restype = ctypes.c_int
_lib.hs2_stream_read_ms.argtypes = [_P, ctypes.c_size_t, _P, ctypes.c_int32, _P,
                                    ctypes.POINTER(ctypes.c_float)]
_lib.hs2_stream_read_ms.restype = ctypes.c_int
# q_full, q_sparse, k, v, out_full, out_sparse, idx, n_sel, lse, scores, stream
_lib.hs2_cross_decoder_step_static.argtypes = [_SP, ctypes.c_int32] + [_P] * 11
_lib.hs2_cross_decoder_step_static.restype = ctypes.c_int
_lib.hs2_status_string.argtypes = [ctypes.c_int]
_lib.hs2_status_string.restype = ctypes.c_char_p
_lib.hs2_last_hip_error.argtypes = []
_lib.hs2_last_hip_error.restype = ctypes.c_int


class HS2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.hs2_status_string(status).decode()
        if status == HS2_ERR_HIP:
            msg += f" (hipError {_lib.hs2_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


@dataclass(frozen=True)
class ShapeArgs:
    batch: int
    n_q_tokens: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    top_k: int = 1024
    window: int = 128
    scale: Optional[float] = None
    kv_capacity: int = 0      # token rows per KV head in k / v; 0 = ctx_len
    select_block: int = 0     # 0: token-level selection; else the block-level variant's block
    decode_splits: int = 0    # 0: the library's plan; else context splits per decode row
    decode_select: int = 0    # 0: the library's plan; 1: from subtile bounds; 2: from every key

    def c(self) -> Shape:
        scale = self.scale if self.scale is not None else 1.0 / math.sqrt(self.head_dim)
        return Shape(ctx_len=self.ctx_len, scale=scale, batch=self.batch,
                     n_q_tokens=self.n_q_tokens, n_q_heads=self.n_q_heads,
                     n_kv_heads=self.n_kv_heads, head_dim=self.head_dim, top_k=self.top_k,
                     window=self.window, select_block=self.select_block,
                     kv_capacity=self.kv_capacity, decode_splits=self.decode_splits,
                     decode_select=self.decode_select)

    @property
    def rows(self) -> int:
        return self.batch * self.n_q_tokens * self.n_kv_heads

    @property
    def cap(self) -> int:
        return self.top_k + self.window

    @property
    def kv_rows(self) -> int:
        """Token rows per KV head of the k / v tensors."""
        return self.kv_capacity or self.ctx_len


def shape_of(workload) -> ShapeArgs:
    """ShapeArgs of a kv_reuse_amd.workloads.Workload."""
    w = workload
    return ShapeArgs(batch=w.batch, n_q_tokens=w.n_q_tokens, n_q_heads=w.n_q_heads,
                     n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, ctx_len=w.ctx_len,
                     top_k=w.top_k, window=w.window, scale=w.scale)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t: Optional[torch.Tensor], name: str, dtype, shape, allow_none=False):
    if t is None:
        if allow_none:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")


def _call(fn: str, status: int):
    if status != HS2_OK:
        raise HS2Error(fn, status)


def workspace_bytes(s: ShapeArgs, n_sparse_layers: int = 0) -> int:
    return int(_lib.hs2_workspace_bytes(ctypes.byref(s.c()), int(n_sparse_layers)))


def alloc_workspace(s: ShapeArgs, n_sparse_layers: int = 0, device="cuda") -> torch.Tensor:
    n = workspace_bytes(s, n_sparse_layers)
    if n == 0:
        raise HS2Error("hs2_workspace_bytes", HS2_ERR_UNSUPPORTED)
    return torch.empty(n, dtype=torch.uint8, device=device)


HS2_WS_LSE2 = 1
HS2_WS_REFINE = 2
HS2_WS_INDEX_CHECK = 3


def workspace_region(s: ShapeArgs, n_sparse_layers: int, region: int):
    """(offset, bytes) of a named region of the workspace (hs2_workspace_region)."""
    off, nb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _call("hs2_workspace_region", _lib.hs2_workspace_region(
        ctypes.byref(s.c()), int(n_sparse_layers), int(region), ctypes.byref(off),
        ctypes.byref(nb)))
    return int(off.value), int(nb.value)


def workspace_lse2(s: ShapeArgs, n_sparse_layers: int, ws: torch.Tensor) -> torch.Tensor:
    """The base-2 log-normalisers [B][T][Hq] (float64) that a step left in ws."""
    off, nb = workspace_region(s, n_sparse_layers, HS2_WS_LSE2)
    return ws[off:off + nb].view(torch.float64).view(s.batch, s.n_q_tokens, s.n_q_heads)


def workspace_refine_stats(s: ShapeArgs, n_sparse_layers: int, ws: torch.Tensor) -> torch.Tensor:
    """Per-row statistics of the normaliser's refinement [rows][4] (uint32 as
    int32): dominant units summed again; a count expected 0 (float32 replica
    mismatches, or heads whose normaliser moved beyond the selection's bound);
    dominant keys beyond the list (expected 0); for the token-level per-row
    selection (a prefill chunk, or decode with the dense selection) the older
    keys its pass listed (above 8192 a second read of the row finds the band),
    else 0."""
    off, nb = workspace_region(s, n_sparse_layers, HS2_WS_REFINE)
    return ws[off:off + nb].view(torch.int32).view(s.rows, 4)


def workspace_index_check(s: ShapeArgs, n_sparse_layers: int, ws: torch.Tensor) -> torch.Tensor:
    """Per-row count [rows] (int64) of the index-list entries that the last
    sparse layers found outside [0, P_t] (hs2_workspace_region, HS2_WS_INDEX_CHECK)."""
    off, nb = workspace_region(s, n_sparse_layers, HS2_WS_INDEX_CHECK)
    return ws[off:off + nb].view(torch.int32).view(s.rows, -1).to(torch.int64).sum(dim=1)


def full_attn_scores(s: ShapeArgs, q, k, v, out, lse=None, scores=None, ws=None):
    B, T, Hq, Hkv, D, S = s.batch, s.n_q_tokens, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ctx_len
    _check(q, "q", torch.bfloat16, (B, T, Hq, D))
    _check(k, "k", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(out, "out", torch.bfloat16, (B, T, Hq, D))
    _check(lse, "lse", torch.float32, (B, T, Hq), allow_none=True)
    _check(scores, "scores", torch.float32, (B, T, Hkv, S), allow_none=True)
    ws = alloc_workspace(s, 0) if ws is None else ws
    _call("hs2_full_attn_scores", _lib.hs2_full_attn_scores(
        ctypes.byref(s.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(scores),
        _ptr(ws), ws.numel(), _stream()))


def topk_select(s: ShapeArgs, scores, idx, n_sel, ws=None):
    B, T, Hkv, S = s.batch, s.n_q_tokens, s.n_kv_heads, s.ctx_len
    _check(scores, "scores", torch.float32, (B, T, Hkv, S))
    _check(idx, "idx", torch.int32, (B, T, Hkv, s.cap))
    _check(n_sel, "n_sel", torch.int32, (B, T, Hkv))
    ws = alloc_workspace(s, 0) if ws is None else ws
    _call("hs2_topk_select", _lib.hs2_topk_select(
        ctypes.byref(s.c()), _ptr(scores), _ptr(idx), _ptr(n_sel), _ptr(ws), ws.numel(),
        _stream()))


def sparse_attn(s: ShapeArgs, q, k, v, idx, n_sel, out, ws=None):
    B, T, Hq, Hkv, D, S = s.batch, s.n_q_tokens, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ctx_len
    L = q.shape[0]
    _check(q, "q", torch.bfloat16, (L, B, T, Hq, D))
    _check(k, "k", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(idx, "idx", torch.int32, (B, T, Hkv, s.cap))
    _check(n_sel, "n_sel", torch.int32, (B, T, Hkv))
    _check(out, "out", torch.bfloat16, (L, B, T, Hq, D))
    ws = alloc_workspace(s, L) if ws is None else ws
    _call("hs2_sparse_attn", _lib.hs2_sparse_attn(
        ctypes.byref(s.c()), L, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(n_sel), _ptr(out),
        _ptr(ws), ws.numel(), _stream()))


def cross_decoder_step(s: ShapeArgs, q_full, q_sparse, k, v, out_full, out_sparse, idx, n_sel,
                       lse=None, scores=None, ws=None):
    B, T, Hq, Hkv, D, S = s.batch, s.n_q_tokens, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ctx_len
    L = 0 if q_sparse is None else q_sparse.shape[0]
    _check(q_full, "q_full", torch.bfloat16, (B, T, Hq, D))
    _check(k, "k", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(out_full, "out_full", torch.bfloat16, (B, T, Hq, D))
    if L:
        _check(q_sparse, "q_sparse", torch.bfloat16, (L, B, T, Hq, D))
        _check(out_sparse, "out_sparse", torch.bfloat16, (L, B, T, Hq, D))
    _check(idx, "idx", torch.int32, (B, T, Hkv, s.cap))
    _check(n_sel, "n_sel", torch.int32, (B, T, Hkv))
    _check(lse, "lse", torch.float32, (B, T, Hq), allow_none=True)
    _check(scores, "scores", torch.float32, (B, T, Hkv, S), allow_none=True)
    ws = alloc_workspace(s, L) if ws is None else ws
    _call("hs2_cross_decoder_step", _lib.hs2_cross_decoder_step(
        ctypes.byref(s.c()), L, _ptr(q_full), _ptr(q_sparse), _ptr(k), _ptr(v), _ptr(out_full),
        _ptr(out_sparse), _ptr(idx), _ptr(n_sel), _ptr(lse), _ptr(scores), _ptr(ws), ws.numel(),
        _stream()))


def cross_decoder_step_static(s: ShapeArgs, q_full, q_sparse, k, v, out_full, out_sparse, idx,
                              n_sel, lse=None, scores=None):
    """cross_decoder_step on the library-held device buffer: no workspace, no
    allocation (hs2_cross_decoder_step_static).  Calls that overlap on one GPU
    share that buffer and race."""
    B, T, Hq, Hkv, D, S = s.batch, s.n_q_tokens, s.n_q_heads, s.n_kv_heads, s.head_dim, s.ctx_len
    L = 0 if q_sparse is None else q_sparse.shape[0]
    _check(q_full, "q_full", torch.bfloat16, (B, T, Hq, D))
    _check(k, "k", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(out_full, "out_full", torch.bfloat16, (B, T, Hq, D))
    if L:
        _check(q_sparse, "q_sparse", torch.bfloat16, (L, B, T, Hq, D))
        _check(out_sparse, "out_sparse", torch.bfloat16, (L, B, T, Hq, D))
    _check(idx, "idx", torch.int32, (B, T, Hkv, s.cap))
    _check(n_sel, "n_sel", torch.int32, (B, T, Hkv))
    _check(lse, "lse", torch.float32, (B, T, Hq), allow_none=True)
    _check(scores, "scores", torch.float32, (B, T, Hkv, S), allow_none=True)
    _call("hs2_cross_decoder_step_static", _lib.hs2_cross_decoder_step_static(
        ctypes.byref(s.c()), L, _ptr(q_full), _ptr(q_sparse), _ptr(k), _ptr(v), _ptr(out_full),
        _ptr(out_sparse), _ptr(idx), _ptr(n_sel), _ptr(lse), _ptr(scores), _stream()))


def cross_decoder_step_timed(s: ShapeArgs, q_full, q_sparse, k, v, out_full, out_sparse, idx,
                             n_sel, ws, iters: int):
    """Per-phase average milliseconds [full split kernel, combine, selection, sparse]."""
    L = 0 if q_sparse is None else q_sparse.shape[0]
    ms = (ctypes.c_float * 4)()
    _call("hs2_cross_decoder_step_timed", _lib.hs2_cross_decoder_step_timed(
        ctypes.byref(s.c()), L, _ptr(q_full), _ptr(q_sparse), _ptr(k), _ptr(v), _ptr(out_full),
        _ptr(out_sparse), _ptr(idx), _ptr(n_sel), _ptr(ws), ws.numel(), _stream(), int(iters), ms))
    return [float(x) for x in ms]


def stream_read_ms(buf: torch.Tensor, iters: int) -> float:
    """Average milliseconds per non-temporal streaming read of the whole of buf
    (a contiguous device tensor); synchronises the current stream."""
    if buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    ms = ctypes.c_float(0.0)
    _call("hs2_stream_read_ms", _lib.hs2_stream_read_ms(
        _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(iters), _stream(),
        ctypes.byref(ms)))
    return float(ms.value)


def raw():
    """The ctypes library handle (for ABI tests)."""
    return _lib


def kv_bridge(hidden, w_kv, k, v, pos0: int):
    """KV Bridging into the cache: hidden [B][n][d_model] and w_kv
    [2][Hkv][D][d_model] (bf16) write rows pos0 .. pos0 + n - 1 of every KV head
    of the caches k, v [B][Hkv][capacity][D]."""
    B, n, dm = hidden.shape
    _, Hkv, D, _ = w_kv.shape
    cap = k.shape[2]
    _check(hidden, "hidden", torch.bfloat16, (B, n, dm))
    _check(w_kv, "w_kv", torch.bfloat16, (2, Hkv, D, dm))
    _check(k, "k", torch.bfloat16, (B, Hkv, cap, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, cap, D))
    sh = BridgeShape(kv_capacity=cap, pos0=int(pos0), batch=B, n_tokens=n, d_model=dm,
                     n_kv_heads=Hkv, head_dim=D, reserved=0)
    _call("hs2_kv_bridge", _lib.hs2_kv_bridge(ctypes.byref(sh), _ptr(hidden), _ptr(w_kv), _ptr(k),
                                              _ptr(v), _stream()))


def local_rows(s: ShapeArgs) -> int:
    """Rows of each layer's local window cache for the separate-window variant."""
    return min(s.ctx_len, s.n_q_tokens + s.window - 1)


def sparse_attn_swa(s: ShapeArgs, q, k, v, idx, n_sel, k_loc, v_loc, out, ws=None):
    """The separate sliding-window branch variant of the sparse layers."""
    B, T, Hq, Hkv, D = s.batch, s.n_q_tokens, s.n_q_heads, s.n_kv_heads, s.head_dim
    L = q.shape[0]
    Lc = local_rows(s)
    _check(q, "q", torch.bfloat16, (L, B, T, Hq, D))
    _check(k, "k", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(v, "v", torch.bfloat16, (B, Hkv, s.kv_rows, D))
    _check(idx, "idx", torch.int32, (B, T, Hkv, s.cap))
    _check(n_sel, "n_sel", torch.int32, (B, T, Hkv))
    # with no local rows (w = 0 in decode) the caches may be None
    _check(k_loc, "k_loc", torch.bfloat16, (L, B, Hkv, Lc, D), allow_none=Lc == 0)
    _check(v_loc, "v_loc", torch.bfloat16, (L, B, Hkv, Lc, D), allow_none=Lc == 0)
    _check(out, "out", torch.bfloat16, (L, B, T, Hq, D))
    ws = alloc_workspace(s, L) if ws is None else ws
    _call("hs2_sparse_attn_swa", _lib.hs2_sparse_attn_swa(
        ctypes.byref(s.c()), L, _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(n_sel), _ptr(k_loc),
        _ptr(v_loc), _ptr(out), _ptr(ws), ws.numel(), _stream()))
