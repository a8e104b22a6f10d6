"""The fused indexer -> top-k (dsa_indexer_topk, and dsa_forward where it fuses) against the unfused
path: the selected index lists must equal dsa_topk's on dsa_indexer_scores' output bit for bit (that
path is itself checked against the oracle's top-k in test_gpu_parity.py), and a few rows are checked
against the oracle directly.

Cases cover one and two queries per sequence, contiguous caches and pages of 64 and 16 tokens, rows
shorter than k (every position selected), rows that end inside a slice or a 32-key subtile, sequences
shorter than a slice, rows short enough for one workgroup to select them whole (no merge pass), rows
that fit one workgroup but are split into slices of at least 8192 positions because one workgroup
per sequence would leave CUs idle, and shapes that do not qualify for the fused pass (bf16, 48
heads), which take the scores through the workspace instead.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import NTHREADS, log, sets
from sparse_attention_sum_amd import dsa, synth
from sparse_attention_sum_amd.device import to_device

pytestmark = pytest.mark.gpu

CASES = [
    # name, ctx, nq, idx heads, dtype, paged, page size
    ("fused-1q-contig", [131072, 100000, 70001, 40000], [1, 1, 1, 1], 64, synth.FP8, False, 64),
    ("fused-2q-paged64", [70000, 65537, 50000], [2, 2, 1], 64, synth.FP8, True, 64),
    ("fused-1q-h32-page16-short-rows", [40000, 2000, 33000, 1500, 90000], [1] * 5, 32, synth.FP8, True, 16),
    ("fused-2q-h32-contig", [36000, 33333], [2, 2], 32, synth.FP8, False, 64),
    ("row-1q-contig", [8192] * 4 + [3000, 8000], [1] * 6, 64, synth.FP8, False, 64),
    ("split-1q-contig-mid", [20000, 17000, 3000, 32768], [1] * 4, 64, synth.FP8, False, 64),
    ("split-1q-paged64-mid", [24576, 16385, 900], [1] * 3, 64, synth.FP8, True, 64),
    ("row-2q-paged64", [16000, 9000, 500], [2, 2, 1], 64, synth.FP8, True, 64),
    ("split-1q-h32-page16", [32768, 2049, 2048, 100], [1] * 4, 32, synth.FP8, True, 16),
    ("unfused-bf16", [40000, 9000], [1, 1], 64, synth.BF16, False, 64),
    ("unfused-h48", [50000, 700], [1, 1], 48, synth.FP8, True, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_indexer_topk_equals_scores_then_topk(case):
    name, ctx, nq, hi, dt, paged, ps = case
    spec = synth.Spec(name, ctx=ctx, nq=nq, idx_heads=hi, idx_dtype=dt, topk=2048, mla_heads=8, paged=paged,
                      page_size=ps, seed=71)
    p = synth.build(spec)
    dp = to_device(p)
    b = dp.batch
    ld = dsa.score_ld(b)
    log(f"{name}: T={spec.T} max_len={p.max_len}")
    scores = dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, scale=spec.idx_scale, ld=ld)
    want = dsa.dsa_topk(scores, ld, b, spec.topk)
    got = dsa.dsa_indexer_topk(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, spec.topk, scale=spec.idx_scale)
    torch.cuda.synchronize()
    assert torch.equal(got, want), f"{name}: fused selection differs from the unfused one"
    # two rows against the oracle's top-k on the GPU's scores
    rows = np.array([0, spec.T - 1], dtype=np.int32)
    g = scores[torch.from_numpy(rows).long().cuda()].cpu().numpy().astype(np.float64)
    ref = oracle.topk(g, p.q_len, spec.topk, rows=rows, nthreads=NTHREADS)
    assert sets(got[torch.from_numpy(rows).long().cuda()].cpu().numpy()) == sets(ref)
    log(f"{name}: fused == unfused on {spec.T} rows, oracle rows ok")


def test_forward_fused_at_full_decode_size_equals_the_chain():
    """decode 64 x 131072 (inputs drawn on the device): dsa_forward takes the fused pass there; its
    indices, output and lse must equal the three separate calls' bit for bit."""
    d = synth.build_decode_on_device(131072, 64, seed=5)
    b = dsa.Batch(cu_q=d["cu_q"], q_seq=d["q_seq"], q_len=d["q_len"], max_len=131072, max_q=1)
    kc = dsa.Cache(d["k_idx"], d["k_idx_scale"], seq_stride=131072)
    lc = dsa.Cache(d["latent"], seq_stride=131072)
    T, H, k, scale = 64, 128, 2048, 1.0 / 24.0
    ind = torch.empty((T, k), dtype=torch.int32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out, _, _ = dsa.dsa_forward(d["q_idx"], d["q_idx_scale"], d["w"], kc, k, d["q_mla"], lc, b, scale,
                                indices_out=ind, lse=lse)
    ld = dsa.score_ld(b)
    scores = dsa.dsa_indexer_scores(d["q_idx"], d["q_idx_scale"], d["w"], kc, b, ld=ld)
    idx2 = dsa.dsa_topk(scores, ld, b, k)
    out2, lse2 = dsa.dsa_sparse_mla(d["q_mla"], lc, b, idx2, scale)
    torch.cuda.synchronize()
    assert torch.equal(ind, idx2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)
    log("decode 64 x 131072: fused forward == chain (bitwise)")
