"""Upload a synthetic workload (synth.Problem) to the GPU as libdsa Cache / Batch objects.

Plumbing only: copies host arrays into torch device tensors with the dtype libdsa expects.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import synth
from .dsa import Batch, Cache


@dataclasses.dataclass
class DeviceProblem:
    problem: synth.Problem
    batch: Batch
    q_idx: torch.Tensor
    q_idx_scale: Optional[torch.Tensor]
    w: torch.Tensor
    k_cache: Cache
    q_mla: torch.Tensor
    latent: Cache

    @property
    def spec(self) -> synth.Spec:
        return self.problem.spec


def _typed(a: np.ndarray, kind: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if kind == synth.BF16:
        t = t.view(torch.int16).view(torch.bfloat16)
    elif kind == synth.FP8:
        t = t.view(torch.uint8).view(torch.float8_e4m3fn)
    return t.to(device)


def to_device(p: synth.Problem, device="cuda") -> DeviceProblem:
    s = p.spec
    dev = torch.device(device)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    batch = Batch(cu_q=i32(p.cu_q), q_seq=i32(p.q_seq), q_len=i32(p.q_len), max_len=p.max_len, max_q=p.max_q)
    pt = None if p.page_table is None else i32(p.page_table)
    f32 = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    k_cache = Cache(data=_typed(p.k_idx, s.idx_dtype, dev), scale=f32(p.k_idx_scale), seq_stride=p.seq_stride,
                    page_table=pt, page_size=s.page_size)
    latent = Cache(data=_typed(p.latent, synth.BF16, dev), seq_stride=p.seq_stride, page_table=pt,
                   page_size=s.page_size)
    return DeviceProblem(problem=p, batch=batch, q_idx=_typed(p.q_idx, s.idx_dtype, dev),
                         q_idx_scale=f32(p.q_idx_scale), w=f32(p.w), k_cache=k_cache,
                         q_mla=_typed(p.q_mla, synth.BF16, dev), latent=latent)
