"""CPU oracle of the DSA hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import this package.
It wraps ``oracle.c`` (plain C, double precision, pthreads over queries) with ctypes and never
imports the GPU library; the two share nothing but the seeded input arrays handed to them.

Each function follows the definition cited in ``oracle.c``:
  * ``indexer``     the lightning indexer's per-head ReLU, weight and head sum, with causal mask;
  * ``topk``        the k best positions per query, ties to the lower position, all when n <= k;
  * ``sparse_mla``  softmax attention of each head over the selected latent rows (MQA form);
  * ``forward``     the three in sequence; the indexer is skipped where n <= k since the selection
                    then does not depend on it;
  * ``topk_select``  per-query k and the union with a sliding window of recent positions;
  * ``value_restore`` each head's value up-projection of the latent attention output (MQA form);
  * ``rope_rows``, ``rope_store``, ``cache_append``, ``bf16_encode``, ``e4m3_encode``: the cache
                    write path (rotary embedding in double, one rounding to binary32, then bf16 or
                    per-row-scaled fp8 storage, and the paged / contiguous append).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "bf16": 1, "fp8": 2}

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, -O2)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC,
                           "-lm", "-lpthread"])
    os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        P, I32, I64, D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        _lib.orc_decode.argtypes = [P, ctypes.c_int, I64, P]
        _lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
        _lib.orc_bf16_value.restype = D
        _lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        _lib.orc_e4m3_value.restype = D
        _lib.orc_indexer.argtypes = [P, ctypes.c_int, P, P, I32, I32, I32,
                                     P, ctypes.c_int, P, I64, P, I32, I32,
                                     P, P, P, I32, D, P, I64, ctypes.c_int]
        _lib.orc_topk.argtypes = [P, I64, I32, P, P, I32, P, ctypes.c_int]
        _lib.orc_topk_select.argtypes = [P, I64, I32, P, P, I32, P, I32, P, ctypes.c_int]
        _lib.orc_value_restore.argtypes = [P, P, I32, I32, I32, P, ctypes.c_int]
        _lib.orc_sparse_mla.argtypes = [P, I32, I32, I32, I32, P, I64, P, I32, I32,
                                        P, P, P, I32, P, I32, D, P, P, ctypes.c_int]
        _lib.orc_bf16_encode.argtypes = [ctypes.c_float]
        _lib.orc_bf16_encode.restype = ctypes.c_uint16
        _lib.orc_e4m3_encode.argtypes = [D]
        _lib.orc_e4m3_encode.restype = ctypes.c_uint8
        I = ctypes.c_int
        _lib.orc_rope_rows.argtypes = [P, I, I64, I, P, I, I, I, D, P]
        _lib.orc_rope_store.argtypes = [P, I, I64, I, I, P, I, I, I, D, P, I, P]
        _lib.orc_cache_append.argtypes = [P, I, I32, I, P, P, I32, I, I, I, D, P, I, P, I64, I64, P, I32, I32]
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact values of raw f32 / bf16-bit / e4m3-bit storage, as float64."""
    raw = _c(raw)
    out = np.empty(raw.shape, dtype=np.float64)
    lib().orc_decode(_ptr(raw), DTYPE_CODE[dtype], raw.size, _ptr(out))
    return out


def indexer(q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_seq, q_len, *, seq_stride=0,
            page_table=None, page_size=64, scale=1.0, ld=None, qsel=None, nthreads=0):
    """Index scores S[r, s] (float64) for query rows qsel (or all), -inf where s >= n_t.

    q: [T, H, D] raw storage; w: float32 [T, H]; q_scale: float32 [T, H] or None;
    k: [rows, D] raw storage; k_scale: float32 [rows] or None; page_table: int32 [B, P] or None.
    """
    q = _c(q); k = _c(k)
    T, H, D = q.shape
    w = _c(w, np.float32); q_scale = _c(q_scale, np.float32); k_scale = _c(k_scale, np.float32)
    q_seq = _c(q_seq, np.int32); q_len = _c(q_len, np.int32)
    pt = _c(page_table, np.int32)
    sel = _c(qsel, np.int32)
    R = T if sel is None else len(sel)
    if ld is None:
        ld = int(q_len.max()) if sel is None else int(q_len[sel].max())
    out = np.empty((R, ld), dtype=np.float64)
    lib().orc_indexer(_ptr(q), DTYPE_CODE[q_dtype], _ptr(q_scale), _ptr(w), T, H, D,
                      _ptr(k), DTYPE_CODE[k_dtype], _ptr(k_scale), int(seq_stride),
                      _ptr(pt), 0 if pt is None else pt.shape[1], int(page_size),
                      _ptr(q_seq), _ptr(q_len), _ptr(sel), 0 if sel is None else len(sel),
                      float(scale), _ptr(out), int(ld), int(nthreads))
    return out


def topk(scores, q_len, k, rows=None, nthreads=0):
    """Top-k positions per score row (row r belongs to query rows[r], or r): int32 [R, k],
    listed best first, -1 padded when n_t < k."""
    s = _c(scores, np.float64)
    R, ld = s.shape
    q_len = _c(q_len, np.int32)
    rows = _c(rows, np.int32)
    out = np.empty((R, k), dtype=np.int32)
    lib().orc_topk(_ptr(s), int(ld), R, _ptr(q_len), _ptr(rows), int(k), _ptr(out), int(nthreads))
    return out


def topk_select(scores, q_len, k, k_per_query=None, window=0, rows=None, nthreads=0):
    """Selection variants: query t's best min(max(k_per_query[t], 0), k) positions (k when None; all
    when n_t is not larger), united with its last `window` positions; int32 [R, k + window] in
    ascending position order, -1 padded."""
    s = _c(scores, np.float64)
    R, ld = s.shape
    q_len = _c(q_len, np.int32)
    rows = _c(rows, np.int32)
    kq = _c(k_per_query, np.int32)
    out = np.empty((R, k + window), dtype=np.int32)
    lib().orc_topk_select(_ptr(s), int(ld), R, _ptr(q_len), _ptr(rows), int(k), _ptr(kq), int(window), _ptr(out),
                          int(nthreads))
    return out


def sparse_mla(q, latent, q_seq, q_len, idx, *, seq_stride=0, page_table=None, page_size=64,
               softmax_scale=1.0 / 24.0, d_v=512, qsel=None, nthreads=0):
    """Sparse MQA-form attention. q: bf16 bits [T, H, Dqk]; latent: bf16 bits [rows, Dqk];
    idx: int32 [R, k] for query rows qsel (or all). Returns (out [R, H, d_v], lse [R, H]) float64."""
    q = _c(q, np.uint16); latent = _c(latent, np.uint16)
    T, H, Dqk = q.shape
    idx = _c(idx, np.int32)
    R, k = idx.shape
    sel = _c(qsel, np.int32)
    assert R == (T if sel is None else len(sel))
    pt = _c(page_table, np.int32)
    out = np.empty((R, H, d_v), dtype=np.float64)
    lse = np.empty((R, H), dtype=np.float64)
    lib().orc_sparse_mla(_ptr(q), T, H, Dqk, int(d_v), _ptr(latent), int(seq_stride),
                         _ptr(pt), 0 if pt is None else pt.shape[1], int(page_size),
                         _ptr(_c(q_seq, np.int32)), _ptr(_c(q_len, np.int32)), _ptr(idx), int(k),
                         _ptr(sel), 0 if sel is None else len(sel),
                         float(softmax_scale), _ptr(out), _ptr(lse), int(nthreads))
    return out, lse


def forward(q_idx, q_idx_dtype, q_idx_scale, w, k_idx, k_idx_dtype, k_idx_scale,
            q_mla, latent, q_seq, q_len, k, *, seq_stride=0, page_table=None, page_size=64,
            scale=1.0, softmax_scale=1.0 / 24.0, d_v=512, qsel=None, nthreads=0):
    """Indexer -> top-k -> sparse MLA for query rows qsel (or all).
    Returns (indices [R, k], out [R, H, d_v], lse [R, H])."""
    q_len = np.ascontiguousarray(q_len, dtype=np.int32)
    T = q_len.shape[0]
    sel = np.arange(T, dtype=np.int32) if qsel is None else np.ascontiguousarray(qsel, dtype=np.int32)
    idx = np.full((len(sel), k), -1, dtype=np.int32)
    long_rows = np.nonzero(q_len[sel] > k)[0]
    short_rows = np.nonzero(q_len[sel] <= k)[0]
    for r in short_rows:                      # context within k: every token, no scoring needed
        idx[r, :q_len[sel[r]]] = np.arange(q_len[sel[r]], dtype=np.int32)
    if len(long_rows):
        lsel = sel[long_rows]
        S = indexer(q_idx, q_idx_dtype, q_idx_scale, w, k_idx, k_idx_dtype, k_idx_scale, q_seq, q_len,
                    seq_stride=seq_stride, page_table=page_table, page_size=page_size, scale=scale,
                    qsel=lsel, nthreads=nthreads)
        idx[long_rows] = topk(S, q_len, k, rows=lsel, nthreads=nthreads)
    out, lse = sparse_mla(q_mla, latent, q_seq, q_len, idx, seq_stride=seq_stride,
                          page_table=page_table, page_size=page_size, softmax_scale=softmax_scale,
                          d_v=d_v, qsel=sel, nthreads=nthreads)
    return idx, out, lse


# --------------------------------------------------------------------------------------------
# cache write path


def bf16_encode(x) -> np.ndarray:
    """bf16 codes (uint16) nearest to binary32 values, ties to the even code."""
    x = np.asarray(x, dtype=np.float32)
    f = lib().orc_bf16_encode
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def e4m3_encode(x) -> np.ndarray:
    """e4m3fn codes (uint8) nearest to values, ties to the even code, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    f = lib().orc_e4m3_encode
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def _rope_args(rope):
    off, d, inter, base = rope if rope is not None else (0, 0, 1, 10000.0)
    return int(off), int(d), int(inter), float(base)


def rope_rows(x, src_dtype: str, pos, rope) -> np.ndarray:
    """Rows x [R, width] (f32 array or bf16 bits) rotated at positions pos [R] in double, rounded
    once to float32.  rope = (offset, dim, interleaved, base)."""
    x = _c(x)
    R, width = x.shape
    pos = _c(pos, np.int32)
    out = np.empty((R, width), dtype=np.float32)
    lib().orc_rope_rows(_ptr(x), DTYPE_CODE[src_dtype], R, width, _ptr(pos), *_rope_args(rope), _ptr(out))
    return out


def rope_store(x, src_dtype: str, pos, rope, dst_dtype: str):
    """Rows x [T, heads, width] rotated at the token positions pos [T] and stored in dst_dtype.
    Returns (stored rows [T, heads, width] as f32 / bf16 bits / e4m3 bits, scales [T, heads] or None)."""
    x = _c(x)
    T, heads, width = x.shape
    pos = _c(pos, np.int32)
    npdt = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dst_dtype]
    out = np.zeros((T, heads, width), dtype=npdt)
    scale = np.zeros((T, heads), dtype=np.float32) if dst_dtype == "fp8" else None
    lib().orc_rope_store(_ptr(x), DTYPE_CODE[src_dtype], T * heads, width, heads, _ptr(pos), *_rope_args(rope),
                         _ptr(out), DTYPE_CODE[dst_dtype], _ptr(scale))
    return out, scale


def cache_append(x, src_dtype: str, seq, pos, num_seqs: int, rope, cache, cache_dtype: str, cache_scale=None,
                 *, seq_stride=0, page_table=None, page_size=64):
    """Append rows x [T, width] to `cache` ([rows, width] numpy storage, modified in place; fp8
    scales go to cache_scale [rows]).  Tokens that map outside the cache are not written."""
    x = _c(x)
    T, width = x.shape
    assert cache.flags["C_CONTIGUOUS"] and cache.shape[1] == width
    seq = _c(seq, np.int32); pos = _c(pos, np.int32)
    pt = _c(page_table, np.int32)
    lib().orc_cache_append(_ptr(x), DTYPE_CODE[src_dtype], T, width, _ptr(seq), _ptr(pos), int(num_seqs),
                           *_rope_args(rope), _ptr(cache), DTYPE_CODE[cache_dtype], _ptr(cache_scale),
                           cache.shape[0], int(seq_stride), _ptr(pt), 0 if pt is None else pt.shape[1],
                           int(page_size))
    return cache


def value_restore(o, w, nthreads=0):
    """o: bf16 bits [T, H, 512]; w: bf16 bits [H, dh, 512].  Returns out [T, H, dh] float64 with
    out[t, h, n] = sum_k o[t, h, k] * w[h, n, k]."""
    o = _c(o, np.uint16); w = _c(w, np.uint16)
    T, H, _ = o.shape
    dh = w.shape[1]
    out = np.empty((T, H, dh), dtype=np.float64)
    lib().orc_value_restore(_ptr(o), _ptr(w), T, H, dh, _ptr(out), int(nthreads))
    return out
