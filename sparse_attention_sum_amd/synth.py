"""Seeded synthetic inputs for the DSA hot path.

This module only draws and stores numbers; it does none of the method's arithmetic.  Both the
GPU library's tests/benchmark and the CPU oracle's tests consume the arrays it returns, so the
two sides always see the very same bytes.

Every workload is a list of sequences.  Sequence ``b`` has ``ctx[b]`` cached tokens, the last
``nq[b]`` of which are query tokens; query ``i`` of the sequence (0-based) sees the causal prefix
``n = ctx[b] - nq[b] + 1 + i`` (a token sees itself).  Prefill is ``nq == ctx``; decode is
``nq == 1``; two-token speculative decode is ``nq == 2``.

Draw order (one ``numpy.random.default_rng(seed)`` stream): ragged lengths (if any), indexer q,
indexer k, indexer weights, MLA q, latent cache, page permutation.

Number formats: bf16 is round-to-nearest-even of the float32 draw; fp8 is OCP e4m3fn with one
float32 scale per 128-wide row, ``scale = max(|row|max, 1e-12) / 448`` and codes
``RNE(x / scale)`` clamped to +-448.  Conversions use torch's CPU casts.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

F32, BF16, FP8 = "f32", "bf16", "fp8"

D_INDEX = 128      # indexer key/query width
D_QK = 576         # latent key width: 512 latent + 64 decoupled-RoPE dims
D_V = 512          # value width: the first 512 latent dims
PAGE = 64          # tokens per cache page


@dataclasses.dataclass
class Spec:
    name: str
    ctx: List[int]                 # cached tokens per sequence (includes the query tokens)
    nq: List[int]                  # query tokens per sequence (the last nq of ctx)
    idx_heads: int = 64
    idx_dtype: str = FP8
    topk: int = 2048
    mla_heads: int = 128
    paged: bool = False
    page_size: int = PAGE
    seed: int = 0
    w_low: float = 0.0             # indexer weights ~ U(w_low, 1)
    mla_sigma: float = 1.0 / 24.0  # MLA q and latent ~ N(0, mla_sigma^2)
    mla_q_sigma: Optional[float] = None   # overrides the MLA q sigma (peaked softmax case)
    idx_scale: float = 1.0
    softmax_scale: float = 1.0 / math.sqrt(576.0)

    @property
    def T(self) -> int:
        return int(sum(self.nq))

    @property
    def B(self) -> int:
        return len(self.ctx)


@dataclasses.dataclass
class Problem:
    spec: Spec
    # batch description
    q_seq: np.ndarray      # int32 [T]
    q_len: np.ndarray      # int32 [T]
    cu_q: np.ndarray       # int32 [B+1]
    max_len: int
    max_q: int
    # indexer operands (raw storage: float32 / uint16 bf16 bits / uint8 e4m3 bits)
    q_idx: np.ndarray      # [T, H_I, 128]
    q_idx_scale: Optional[np.ndarray]   # float32 [T, H_I] (fp8 only)
    w: np.ndarray          # float32 [T, H_I]
    k_idx: np.ndarray      # [rows, 128]
    k_idx_scale: Optional[np.ndarray]   # float32 [rows] (fp8 only)
    # MLA operands
    q_mla: np.ndarray      # uint16 bf16 bits [T, H, 576]
    latent: np.ndarray     # uint16 bf16 bits [rows, 576]
    # cache layout
    seq_stride: int        # contiguous: rows per sequence (0 when paged)
    page_table: Optional[np.ndarray]    # int32 [B, pages_per_seq] when paged


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _fp8_rows(x: np.ndarray):
    """Per-row (last axis) e4m3fn quantisation: returns (uint8 codes, float32 scales)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (np.maximum(amax, np.float32(1e-12)) / np.float32(448.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def _normal(rng, shape, sigma=1.0, chunk=1 << 24) -> np.ndarray:
    """float32 N(0, sigma^2) draws, generated in chunks to bound peak memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            out[s:e] *= np.float32(sigma)
    return out.reshape(shape)


def _encode(rng, shape, dtype, sigma=1.0):
    """Draw N(0, sigma^2) rows and store them in ``dtype``; returns (raw, scale-or-None)."""
    x = _normal(rng, shape, sigma)
    if dtype == F32:
        return x, None
    if dtype == BF16:
        return _bf16_bits(x), None
    if dtype == FP8:
        return _fp8_rows(x)
    raise ValueError(dtype)


def _bf16_chunked(rng, shape, sigma, chunk_rows=1 << 15) -> np.ndarray:
    """bf16 N(0, sigma^2) with the same draws as _normal, converted chunk by chunk."""
    rows = shape[0]
    per_row = int(np.prod(shape[1:]))
    out = np.empty((rows, per_row), dtype=np.uint16)
    for s in range(0, rows, chunk_rows):
        e = min(rows, s + chunk_rows)
        x = rng.standard_normal((e - s) * per_row, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[s:e] = _bf16_bits(x).reshape(e - s, per_row)
    return out.reshape(shape)


def build(spec: Spec) -> Problem:
    rng = np.random.default_rng(spec.seed)
    B, T = spec.B, spec.T
    ctx = [int(c) for c in spec.ctx]
    nq = [int(m) for m in spec.nq]
    assert len(ctx) == len(nq) and all(1 <= m <= c for c, m in zip(ctx, nq))

    q_seq = np.empty(T, dtype=np.int32)
    q_len = np.empty(T, dtype=np.int32)
    cu_q = np.zeros(B + 1, dtype=np.int32)
    t = 0
    for b in range(B):
        for i in range(nq[b]):
            q_seq[t] = b
            q_len[t] = ctx[b] - nq[b] + 1 + i
            t += 1
        cu_q[b + 1] = t

    if spec.paged:
        pages_per_seq = [(c + spec.page_size - 1) // spec.page_size for c in ctx]
        rows = sum(pages_per_seq) * spec.page_size
        seq_stride = 0
    else:
        pages_per_seq = None
        rows = B * max(ctx)
        seq_stride = max(ctx)

    H_I = spec.idx_heads
    q_idx, q_idx_scale = _encode(rng, (T, H_I, D_INDEX), spec.idx_dtype)
    k_idx, k_idx_scale = _encode(rng, (rows, D_INDEX), spec.idx_dtype)
    w = rng.uniform(spec.w_low, 1.0, size=(T, H_I)).astype(np.float32)
    qsig = spec.mla_q_sigma if spec.mla_q_sigma is not None else spec.mla_sigma
    q_mla = _bf16_chunked(rng, (T, spec.mla_heads, D_QK), qsig)
    latent = _bf16_chunked(rng, (rows, D_QK), spec.mla_sigma)

    page_table = None
    if spec.paged:
        total = sum(pages_per_seq)
        perm = rng.permutation(total).astype(np.int32)
        width = max(pages_per_seq)
        page_table = np.zeros((B, width), dtype=np.int32)
        p = 0
        for b in range(B):
            page_table[b, :pages_per_seq[b]] = perm[p:p + pages_per_seq[b]]
            p += pages_per_seq[b]

    return Problem(spec=spec, q_seq=q_seq, q_len=q_len, cu_q=cu_q,
                   max_len=int(q_len.max()), max_q=int(max(nq)),
                   q_idx=q_idx, q_idx_scale=q_idx_scale, w=w, k_idx=k_idx, k_idx_scale=k_idx_scale,
                   q_mla=q_mla, latent=latent, seq_stride=seq_stride, page_table=page_table)


def small_integer_indexer(p: Problem, seed: int = 0) -> Problem:
    """The same workload with small-integer indexer operands: q and k in {-3, ..., 3} (stored in the
    workload's indexer dtype: float32, bf16 or e4m3 codes, all exact), every fp8 scale 1, weights in
    {0, 1/4, 1/2, 1}.  Every product, dot product, weighted ReLU and head sum of the indexer is then a
    multiple of 1/4 below 2^22 in magnitude, so any summation order in binary32 gives the exact value."""
    rng = np.random.default_rng(seed)
    s = p.spec
    qv = rng.integers(-3, 4, size=p.q_idx.shape).astype(np.float32)
    kv = rng.integers(-3, 4, size=p.k_idx.shape).astype(np.float32)
    if s.idx_dtype == F32:
        q_raw, k_raw = qv, kv
    elif s.idx_dtype == BF16:
        q_raw, k_raw = _bf16_bits(qv), _bf16_bits(kv)
    else:
        to8 = lambda x: torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        q_raw, k_raw = to8(qv), to8(kv)
    w = rng.choice(np.array([0.0, 0.25, 0.5, 1.0], np.float32), size=p.w.shape)
    fp8 = s.idx_dtype == FP8
    return dataclasses.replace(
        p, q_idx=q_raw, k_idx=k_raw, w=w,
        q_idx_scale=np.ones(p.q_idx.shape[:2], np.float32) if fp8 else None,
        k_idx_scale=np.ones(p.k_idx.shape[0], np.float32) if fp8 else None,
        spec=dataclasses.replace(s, idx_scale=1.0))


# ----------------------------------------------------------------------------------------------
# the five workloads and their variants


def ragged_lengths(rng, B=16, lo=1000, hi=131072, n_short=3, short_hi=2048) -> List[int]:
    """B lengths: B-n_short log-uniform in [lo, hi] and n_short log-uniform in [lo, short_hi],
    shuffled, rounded to integers (so at least n_short sequences take the full-attention path)."""
    long_ = np.exp(rng.uniform(math.log(lo), math.log(hi), size=B - n_short))
    short = np.exp(rng.uniform(math.log(lo), math.log(short_hi), size=n_short))
    lens = np.concatenate([long_, short])
    rng.shuffle(lens)
    return [int(round(v)) for v in lens]


def named_spec(name: str) -> Spec:
    """The five workloads by name: tiny causal prefill (L = 1024, fp32 indexer, 4 heads), batched decode
    (64 x 8192, fp8), long causal prefill (L = 16384, bf16), two-token decode (32 x 2 at 65536, paged),
    and ragged long-context decode (16 sequences, paged)."""
    if name == "tiny-prefill-L1024":
        return Spec(name, ctx=[1024], nq=[1024], idx_heads=4, idx_dtype=F32, topk=256, mla_heads=8, seed=0)
    if name == "decode-B64-ctx8192":
        return Spec(name, ctx=[8192] * 64, nq=[1] * 64, idx_dtype=FP8, seed=1)
    if name == "prefill-L16384":
        return Spec(name, ctx=[16384], nq=[16384], idx_dtype=BF16, seed=2)
    if name == "mtp-decode-B32x2-ctx65536-paged":
        return Spec(name, ctx=[65536] * 32, nq=[2] * 32, idx_dtype=FP8, paged=True, seed=3)
    if name == "ragged-decode-B16-paged":
        rng = np.random.default_rng(4 + 1000)   # lengths from their own stream, seeded by the workload
        return Spec(name, ctx=ragged_lengths(rng), nq=[1] * 16, idx_dtype=FP8, paged=True, seed=4)
    raise ValueError(name)


NAMED = ("tiny-prefill-L1024", "decode-B64-ctx8192", "prefill-L16384", "mtp-decode-B32x2-ctx65536-paged",
         "ragged-decode-B16-paged")


def sweep_spec(ctx: int, batch: int = 64) -> Spec:
    """Batched-decode shape at a longer context (8K..128K sweep)."""
    return Spec(f"decode-B{batch}-ctx{ctx}", ctx=[ctx] * batch, nq=[1] * batch, idx_dtype=FP8, seed=1)


def build_decode_on_device(ctx: int, batch: int = 64, seed: int = 1, device="cuda"):
    """The batched-decode workload drawn directly in device memory (torch's seeded generator on the
    GPU), for contexts whose host-side draw would take minutes: returns a dict of device tensors with
    the same distributions and storage formats as build() (fp8 indexer keys and queries with one scale
    per 128-wide row, w ~ U(0, 1), MLA q and latent ~ N(0, 1/24^2) in bf16, contiguous caches).
    The host copies the rows it checks; the values differ from build()'s for the same seed."""
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(seed)
    T, rows = batch, batch * ctx

    def fp8_rows(shape):
        x = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        amax = x.abs().amax(dim=-1, keepdim=True)
        scale = torch.clamp(amax, min=1e-12) / 448.0
        codes = torch.clamp(x / scale, -448.0, 448.0).to(torch.float8_e4m3fn)
        return codes, scale.squeeze(-1)

    def bf16_normal(shape, sigma, chunk=1 << 26):
        out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        flat = out.view(-1)
        for s0 in range(0, flat.numel(), chunk):
            e = min(flat.numel(), s0 + chunk)
            flat[s0:e] = (torch.randn(e - s0, generator=g, device=dev) * sigma).to(torch.bfloat16)
        return out

    q_idx, q_idx_scale = fp8_rows((T, 64, D_INDEX))
    k_parts, s_parts = [], []
    for r0 in range(0, rows, 1 << 22):
        c, sc = fp8_rows((min(rows, r0 + (1 << 22)) - r0, D_INDEX))
        k_parts.append(c)
        s_parts.append(sc)
    k_idx, k_idx_scale = torch.cat(k_parts), torch.cat(s_parts)
    w = torch.rand((T, 64), generator=g, device=dev, dtype=torch.float32)
    q_mla = bf16_normal((T, 128, D_QK), 1.0 / 24.0)
    latent = bf16_normal((rows, D_QK), 1.0 / 24.0)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    return dict(ctx=ctx, T=T, B=batch, q_idx=q_idx, q_idx_scale=q_idx_scale, w=w, k_idx=k_idx,
                k_idx_scale=k_idx_scale, q_mla=q_mla, latent=latent, seq_stride=ctx,
                cu_q=i32(list(range(T + 1))), q_seq=i32(list(range(T))), q_len=i32([ctx] * T))


def peaked_spec() -> Spec:
    """Tiny-prefill shapes with MLA q ~ N(0, 72^2): with latent ~ N(0, 1/24^2) and the 1/sqrt(576)
    softmax scale, each logit then has standard deviation 72 * 24 / 24 / 24 = 3, so the softmax is
    far from uniform and the running-max rescaling is exercised."""
    s = named_spec("tiny-prefill-L1024")
    return dataclasses.replace(s, name="tiny-prefill-peaked", mla_q_sigma=72.0)


__all__ = ["Spec", "Problem", "build", "named_spec", "NAMED", "sweep_spec", "peaked_spec", "ragged_lengths", "small_integer_indexer",
           "F32", "BF16", "FP8", "D_INDEX", "D_QK", "D_V", "PAGE"]
