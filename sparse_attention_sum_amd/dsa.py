"""ctypes binding of libdsa's C ABI (include/dsa.h), with the same entry-point names.

This module only marshals arguments: torch tensors supply device pointers and the current HIP
stream, every step of the computation runs in libdsa's kernels.  There is no fallback: if
``libdsa.so`` is missing or cannot be loaded, calls raise.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

# dsa_status
DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
# dsa_dtype
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
# operations for dsa_workspace_size
DSA_OP_INDEXER, DSA_OP_TOPK, DSA_OP_SPARSE_MLA, DSA_OP_FORWARD, DSA_OP_INDEXER_TOPK = 0, 1, 2, 3, 4

EXPORTS = ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla", "dsa_forward", "dsa_workspace_size",
           "dsa_status_string", "dsa_last_error", "dsa_version", "dsa_cache_append", "dsa_rope_queries",
           "dsa_topk_select", "dsa_value_restore", "dsa_forward_noalloc", "dsa_indexer_topk")


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libdsa status {status}: {message}")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("num_rows", ctypes.c_int64), ("seq_stride", ctypes.c_int64),
                ("page_table", ctypes.c_void_p), ("page_table_stride", ctypes.c_int32),
                ("page_size", ctypes.c_int32)]


class _Batch(ctypes.Structure):
    _fields_ = [("num_queries", ctypes.c_int32), ("num_seqs", ctypes.c_int32), ("cu_q", ctypes.c_void_p),
                ("q_seq", ctypes.c_void_p), ("q_len", ctypes.c_void_p), ("max_len", ctypes.c_int32),
                ("max_q", ctypes.c_int32)]


class _Rope(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int32), ("dim", ctypes.c_int32), ("interleaved", ctypes.c_int32),
                ("base", ctypes.c_double)]


@dataclasses.dataclass
class Rope:
    """Rotation of the span [offset, offset + dim) of a row: pair i turns by position * base^(-2i/dim);
    pairs are adjacent (interleaved) or the two halves of the span."""
    offset: int = 0
    dim: int = 0
    interleaved: bool = True
    base: float = 10000.0

    def struct(self) -> _Rope:
        return _Rope(int(self.offset), int(self.dim), 1 if self.interleaved else 0, float(self.base))


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libdsa.so (built in-tree by sparse_attention_sum_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m sparse_attention_sum_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    CP, BP = ctypes.POINTER(_Cache), ctypes.POINTER(_Batch)
    L.dsa_indexer_scores.argtypes = [P, I32, P, P, I32, I32, CP, BP, F, P, I64, P]
    L.dsa_topk.argtypes = [P, I64, BP, I32, P, P, ctypes.c_size_t, P]
    L.dsa_indexer_topk.argtypes = [P, I32, P, P, I32, I32, CP, BP, F, I32, P, P, ctypes.c_size_t, P]
    L.dsa_topk_select.argtypes = [P, I64, BP, I32, P, I32, P, P, ctypes.c_size_t, P]
    L.dsa_value_restore.argtypes = [P, P, I32, I32, I32, P, P]
    L.dsa_sparse_mla.argtypes = [P, I32, I32, I32, CP, BP, P, I32, F, P, P, P, ctypes.c_size_t, P]
    L.dsa_forward.argtypes = [P, I32, P, P, I32, CP, F, I32, P, I32, CP, F, BP, P, P, P, P, ctypes.c_size_t, P]
    L.dsa_forward_noalloc.argtypes = [P, I32, P, P, I32, CP, F, I32, P, I32, CP, F, BP, P, P, P, P]
    L.dsa_workspace_size.argtypes = [I32, BP, I32, I32, I32]
    RP = ctypes.POINTER(_Rope)
    L.dsa_cache_append.argtypes = [P, I32, P, I32, P, P, I32, I32, RP, RP, CP, CP, P]
    L.dsa_rope_queries.argtypes = [P, I32, I32, P, I32, P, RP, P, I32, RP, P, I32, P]
    L.dsa_workspace_size.restype = ctypes.c_size_t
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_version.restype = ctypes.c_char_p
    for name in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla", "dsa_forward", "dsa_cache_append",
                 "dsa_rope_queries", "dsa_topk_select", "dsa_value_restore", "dsa_forward_noalloc",
                 "dsa_indexer_topk"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, load().dsa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DSA_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DSA_FP8_E4M3
    raise TypeError(f"no libdsa dtype for {t.dtype}")


@dataclasses.dataclass
class Cache:
    """A token cache: contiguous (seq_stride rows per sequence) or paged (page_table)."""
    data: torch.Tensor                         # [rows, dim]
    scale: Optional[torch.Tensor] = None       # float32 [rows] (fp8)
    seq_stride: int = 0
    page_table: Optional[torch.Tensor] = None  # int32 [B, P]
    page_size: int = 64
    dtype: Optional[int] = None

    def struct(self) -> _Cache:
        return _Cache(self.data.data_ptr(), None if self.scale is None else self.scale.data_ptr(),
                      dtype_code(self.data) if self.dtype is None else self.dtype, int(self.data.shape[-1]),
                      int(self.data.shape[0]), int(self.seq_stride),
                      None if self.page_table is None else self.page_table.data_ptr(),
                      0 if self.page_table is None else int(self.page_table.shape[1]), int(self.page_size))


@dataclasses.dataclass
class Batch:
    """Query tokens grouped by sequence: cu_q [B+1], q_seq [T], q_len [T] (int32 device tensors)."""
    cu_q: torch.Tensor
    q_seq: torch.Tensor
    q_len: torch.Tensor
    max_len: int
    max_q: int

    @property
    def num_queries(self) -> int:
        return int(self.q_len.shape[0])

    def struct(self) -> _Batch:
        return _Batch(self.num_queries, int(self.cu_q.shape[0]) - 1, self.cu_q.data_ptr(), self.q_seq.data_ptr(),
                      self.q_len.data_ptr(), int(self.max_len), int(self.max_q))


def score_ld(batch: Batch) -> int:
    """Row stride of score buffers used by dsa_forward (max_len rounded up to 64)."""
    return (int(batch.max_len) + 63) // 64 * 64


def dsa_workspace_size(op: int, batch: Batch, k: int, n_heads: int, d_v: int = 512) -> int:
    b = batch.struct()
    return int(load().dsa_workspace_size(op, ctypes.byref(b), int(k), int(n_heads), int(d_v)))


def dsa_indexer_scores(q: torch.Tensor, q_scale: Optional[torch.Tensor], weights: torch.Tensor, k_cache: Cache,
                       batch: Batch, scale: float = 1.0, scores: Optional[torch.Tensor] = None,
                       ld: Optional[int] = None, stream=None) -> torch.Tensor:
    """q [T, H, 128]; returns scores [T, ld] float32 (entries s >= n_t are -inf, written by libdsa)."""
    T, H, D = q.shape
    if ld is None:
        ld = score_ld(batch)
    if scores is None:
        scores = torch.empty((T, ld), dtype=torch.float32, device=q.device)
    kc, b = k_cache.struct(), batch.struct()
    _check(load().dsa_indexer_scores(_ptr(q), dtype_code(q), _ptr(q_scale), _ptr(weights), H, D, ctypes.byref(kc),
                                      ctypes.byref(b), float(scale), _ptr(scores), int(ld), _stream(stream)))
    return scores


def dsa_indexer_topk(q: torch.Tensor, q_scale: Optional[torch.Tensor], weights: torch.Tensor, k_cache: Cache,
                     batch: Batch, k: int, scale: float = 1.0, indices: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The indexer and the top-k in one call (fused for long fp8 decode rows); returns indices [T, k]
    int32, ascending positions then -1 -- the same as dsa_topk on dsa_indexer_scores' output."""
    T, H, D = q.shape
    if indices is None:
        indices = torch.empty((T, k), dtype=torch.int32, device=q.device)
    if workspace is None:
        need = dsa_workspace_size(DSA_OP_INDEXER_TOPK, batch, k, H)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need > 0 else None
    kc, b = k_cache.struct(), batch.struct()
    _check(load().dsa_indexer_topk(_ptr(q), dtype_code(q), _ptr(q_scale), _ptr(weights), H, D, ctypes.byref(kc),
                                    ctypes.byref(b), float(scale), int(k), _ptr(indices), _ptr(workspace),
                                    0 if workspace is None else workspace.numel(), _stream(stream)))
    return indices


def _topk_workspace(batch: Batch, k: int, workspace, device):
    """A workspace for the two-pass path of long rows (None when the call needs none)."""
    if workspace is not None:
        return workspace
    need = dsa_workspace_size(DSA_OP_TOPK, batch, k, 1)
    return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None


def dsa_topk(scores: Optional[torch.Tensor], ld: int, batch: Batch, k: int, indices: Optional[torch.Tensor] = None,
             stream=None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Returns indices [T, k] int32: selected positions ascending, then -1."""
    if indices is None:
        indices = torch.empty((batch.num_queries, k), dtype=torch.int32, device=batch.q_len.device)
    ws = _topk_workspace(batch, k, workspace, batch.q_len.device)
    b = batch.struct()
    _check(load().dsa_topk(_ptr(scores), int(ld), ctypes.byref(b), int(k), _ptr(indices), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream(stream)))
    return indices


def dsa_topk_select(scores: torch.Tensor, ld: int, batch: Batch, k: int, k_per_query: Optional[torch.Tensor] = None,
                    window: int = 0, indices: Optional[torch.Tensor] = None, stream=None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-query k (int32 [T] or None) and the union with the last `window` positions; returns int32
    [T, k + window], ascending positions then -1."""
    T = batch.num_queries
    if indices is None:
        indices = torch.empty((T, k + window), dtype=torch.int32, device=scores.device)
    ws = _topk_workspace(batch, k, workspace, scores.device)
    b = batch.struct()
    _check(load().dsa_topk_select(_ptr(scores), int(ld), ctypes.byref(b), int(k), _ptr(k_per_query), int(window),
                                  _ptr(indices), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return indices


def dsa_sparse_mla(q: torch.Tensor, latent: Cache, batch: Batch, indices: torch.Tensor, softmax_scale: float,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, want_lse: bool = True, stream=None):
    """q [T, H, 576] bf16; returns (out [T, H, 512] bf16, lse [T, H] float32 or None)."""
    T, H, Dqk = q.shape
    k = int(indices.shape[1])
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = dsa_workspace_size(DSA_OP_SPARSE_MLA, batch, k, H)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    lc, b = latent.struct(), batch.struct()
    _check(load().dsa_sparse_mla(_ptr(q), H, Dqk, 512, ctypes.byref(lc), ctypes.byref(b), _ptr(indices), k,
                                  float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _stream(stream)))
    return out, lse


def dsa_forward(q_idx: torch.Tensor, q_idx_scale: Optional[torch.Tensor], weights: torch.Tensor, k_cache: Cache,
                k: int, q: torch.Tensor, latent: Cache, batch: Batch, softmax_scale: float, idx_scale: float = 1.0,
                indices_out: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Indexer -> top-k -> sparse MLA.  Returns (out, lse, indices_out)."""
    T, H, _ = q.shape
    HI = int(q_idx.shape[1])
    if out is None:
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        need = dsa_workspace_size(DSA_OP_FORWARD, batch, k, H)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    kc, lc, b = k_cache.struct(), latent.struct(), batch.struct()
    _check(load().dsa_forward(_ptr(q_idx), dtype_code(q_idx), _ptr(q_idx_scale), _ptr(weights), HI,
                               ctypes.byref(kc), float(idx_scale), int(k), _ptr(q), H, ctypes.byref(lc),
                               float(softmax_scale), ctypes.byref(b), _ptr(indices_out), _ptr(out), _ptr(lse),
                               _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse, indices_out


def dsa_forward_noalloc(q_idx: torch.Tensor, q_idx_scale: Optional[torch.Tensor], weights: torch.Tensor,
                        k_cache: Cache, k: int, q: torch.Tensor, latent: Cache, batch: Batch, softmax_scale: float,
                        out: torch.Tensor, idx_scale: float = 1.0, indices_out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None):
    """dsa_forward without a workspace (libdsa's static scratch); out [T, H, 512] bf16 must be given,
    since this call allocates nothing.  Returns (out, lse, indices_out)."""
    T, H, _ = q.shape
    HI = int(q_idx.shape[1])
    kc, lc, b = k_cache.struct(), latent.struct(), batch.struct()
    _check(load().dsa_forward_noalloc(_ptr(q_idx), dtype_code(q_idx), _ptr(q_idx_scale), _ptr(weights), HI,
                                      ctypes.byref(kc), float(idx_scale), int(k), _ptr(q), H, ctypes.byref(lc),
                                      float(softmax_scale), ctypes.byref(b), _ptr(indices_out), _ptr(out), _ptr(lse),
                                      _stream(stream)))
    return out, lse, indices_out


def dsa_cache_append(k_new: Optional[torch.Tensor], latent_new: Optional[torch.Tensor], seq: torch.Tensor,
                     pos: torch.Tensor, num_seqs: int, k_cache: Optional[Cache], latent: Optional[Cache],
                     k_rope: Optional[Rope] = None, latent_rope: Optional[Rope] = None, stream=None):
    """Rotate new tokens' indexer keys [T, 128] and latent rows [T, 576] (f32 or bf16) at positions pos
    [T] and write them into the caches (token i at position pos[i] of sequence seq[i])."""
    T = int(seq.shape[0])
    kc = None if k_cache is None else k_cache.struct()
    lc = None if latent is None else latent.struct()
    kr = None if k_rope is None else k_rope.struct()
    lr = None if latent_rope is None else latent_rope.struct()
    _check(load().dsa_cache_append(_ptr(k_new), DSA_F32 if k_new is None else dtype_code(k_new), _ptr(latent_new),
                                   DSA_F32 if latent_new is None else dtype_code(latent_new), _ptr(seq), _ptr(pos),
                                   T, int(num_seqs), None if kr is None else ctypes.byref(kr),
                                   None if lr is None else ctypes.byref(lr), None if kc is None else ctypes.byref(kc),
                                   None if lc is None else ctypes.byref(lc), _stream(stream)))


def dsa_rope_queries(q_idx_in: Optional[torch.Tensor], q_idx_out: Optional[torch.Tensor],
                     q_idx_scale_out: Optional[torch.Tensor], q_mla: Optional[torch.Tensor], pos: torch.Tensor,
                     idx_rope: Optional[Rope] = None, mla_rope: Optional[Rope] = None, stream=None):
    """Rotate indexer queries [T, H_I, 128] (f32 / bf16) into q_idx_out (f32 / bf16 / fp8 bits with
    row scales in q_idx_scale_out [T, H_I]) and MLA queries [T, H, 576] bf16 in place."""
    T = int(pos.shape[0])
    ir = None if idx_rope is None else idx_rope.struct()
    mr = None if mla_rope is None else mla_rope.struct()
    _check(load().dsa_rope_queries(_ptr(q_idx_in), DSA_F32 if q_idx_in is None else dtype_code(q_idx_in),
                                   0 if q_idx_in is None else int(q_idx_in.shape[1]), _ptr(q_idx_out),
                                   DSA_F32 if q_idx_out is None else dtype_code(q_idx_out), _ptr(q_idx_scale_out),
                                   None if ir is None else ctypes.byref(ir), _ptr(q_mla),
                                   0 if q_mla is None else int(q_mla.shape[1]),
                                   None if mr is None else ctypes.byref(mr), _ptr(pos), T, _stream(stream)))


def dsa_value_restore(latent_out: torch.Tensor, w_uv: torch.Tensor, out: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """latent_out [T, H, 512] bf16, w_uv [H, d_h, 512] bf16 -> out [T, H, d_h] bf16 (each head's value
    up-projection of the latent attention output)."""
    T, H, _ = latent_out.shape
    dh = int(w_uv.shape[1])
    if out is None:
        out = torch.empty((T, H, dh), dtype=torch.bfloat16, device=latent_out.device)
    _check(load().dsa_value_restore(_ptr(latent_out), _ptr(w_uv), T, H, dh, _ptr(out), _stream(stream)))
    return out
