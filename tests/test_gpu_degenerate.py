"""Degenerate batches through the public entry points.

- An empty batch (no query tokens) through every call of the path: nothing is launched and every call
  returns DSA_OK.
- Queries that see no position (n_t = 0) and queries that see fewer positions than k, through
  dsa_forward: with n_t <= k every position is selected (page "一文讀懂DeepSeek-V3.2核心技術DSA",
  "DSA 的四步工作流程", the top-k step keeps all tokens when the context is at most k), in ascending
  order and padded with -1; with n_t = 0 nothing is selected, and the attention output over an empty
  set is 0 with lse = -inf (the library's stated convention for an empty selection).
- k = 1: softmax over a single selected row is exactly 1, so each head's output is that row's first
  512 latent values, bit for bit, and lse is the row's scaled logit.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import NTHREADS, log, oracle_mla, check_mla
from sparse_attention_sum_amd import dsa, synth
from sparse_attention_sum_amd.device import to_device

pytestmark = pytest.mark.gpu


def _device(spec):
    p = synth.build(spec)
    return p, to_device(p)


def test_empty_batch_through_every_entry_point():
    p, dp = _device(synth.Spec("empty-src", ctx=[300], nq=[1], idx_heads=64, idx_dtype=synth.FP8, topk=64,
                               mla_heads=16, seed=3))
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    for max_len in (0, 300):
        b = dsa.Batch(cu_q=torch.zeros(2, dtype=torch.int32, device="cuda"), q_seq=z, q_len=z, max_len=max_len,
                      max_q=1)
        q_idx = dp.q_idx[:0]
        q_sc = dp.q_idx_scale[:0]
        w = dp.w[:0]
        q = dp.q_mla[:0]
        ld = max(64, dsa.score_ld(b))
        scores = torch.empty((0, ld), dtype=torch.float32, device="cuda")
        dsa.dsa_indexer_scores(q_idx, q_sc, w, dp.k_cache, b, scores=scores, ld=ld)
        idx = dsa.dsa_topk(scores, ld, b, 64)
        assert idx.shape == (0, 64)
        idx2 = dsa.dsa_indexer_topk(q_idx, q_sc, w, dp.k_cache, b, 64)
        assert idx2.shape == (0, 64)
        out, lse, _ = dsa.dsa_forward(q_idx, q_sc, w, dp.k_cache, 64, q, dp.latent, b, 1 / 24)
        assert out.shape == (0, 16, 512)
        out_na = torch.empty((0, 16, 512), dtype=torch.bfloat16, device="cuda")
        dsa.dsa_forward_noalloc(q_idx, q_sc, w, dp.k_cache, 64, q, dp.latent, b, 1 / 24, out=out_na)
        torch.cuda.synchronize()
        log(f"empty batch, max_len {max_len}: every entry point returned DSA_OK")


@pytest.mark.parametrize("paged", [False, True])
def test_queries_with_no_or_few_positions(paged):
    k = 64
    spec = synth.Spec(f"few-{paged}", ctx=[3000, 40, 64, 65, 7], nq=[1, 1, 1, 1, 1], idx_heads=64,
                      idx_dtype=synth.FP8, topk=k, mla_heads=16, paged=paged, seed=11)
    p, dp = _device(spec)
    q_len = p.q_len.copy()
    q_len[4] = 0                                   # the last query sees no position
    b = dsa.Batch(cu_q=dp.batch.cu_q, q_seq=dp.batch.q_seq, q_len=torch.from_numpy(q_len).cuda(),
                  max_len=p.max_len, max_q=p.max_q)
    T, H = spec.T, spec.mla_heads
    ind = torch.full((T, k), 12345, dtype=torch.int32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out, _, _ = dsa.dsa_forward(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, k, dp.q_mla, dp.latent, b,
                                spec.softmax_scale, idx_scale=spec.idx_scale, indices_out=ind, lse=lse)
    torch.cuda.synchronize()
    gi = ind.cpu().numpy()
    for t in range(T):
        n = int(q_len[t])
        if n <= k:
            want = np.concatenate([np.arange(n), np.full(k - n, -1)]).astype(np.int32)
            assert np.array_equal(gi[t], want), f"query {t} (n = {n}): {gi[t][:8]} ..."
    # the long row: the selected set against the oracle's top-k on the GPU's own scores
    ld = dsa.score_ld(b)
    scores = dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, scale=spec.idx_scale, ld=ld)
    g = scores[0:1].double().cpu().numpy()
    want = oracle.topk(g, q_len[:1], k, nthreads=NTHREADS)[0]
    assert sorted(gi[0].tolist()) == sorted(want.tolist())
    # attention against the oracle on the GPU's indices; the empty query gives 0 and -inf
    p.q_len = q_len
    o_ref, l_ref = oracle_mla(p, gi)
    check_mla(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"few positions, paged={paged}")
    assert torch.all(out[4] == 0) and torch.all(torch.isneginf(lse[4]))
    log(f"paged={paged}: n <= k rows select 0..n-1 in order, the n = 0 query gives 0 / -inf")


def test_k_one_outputs_the_selected_row_exactly():
    k = 1
    spec = synth.Spec("k1", ctx=[500, 2000, 1], nq=[2, 1, 1], idx_heads=32, idx_dtype=synth.FP8, topk=k,
                      mla_heads=32, seed=13)
    p, dp = _device(spec)
    T, H = spec.T, spec.mla_heads
    ind = torch.empty((T, k), dtype=torch.int32, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    out, _, _ = dsa.dsa_forward(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, k, dp.q_mla, dp.latent, dp.batch,
                                spec.softmax_scale, idx_scale=spec.idx_scale, indices_out=ind, lse=lse)
    torch.cuda.synchronize()
    gi = ind.cpu().numpy()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for t in range(T):
        s = int(gi[t, 0])
        assert 0 <= s < int(p.q_len[t])
        row = p.latent[int(p.q_seq[t]) * p.seq_stride + s]           # uint16 bf16 bits, 576 dims
        assert np.array_equal(o[t], np.broadcast_to(row[:512], (H, 512))), f"query {t}"
    o_ref, l_ref = oracle_mla(p, gi)
    assert np.abs(lse.cpu().numpy() - l_ref).max() <= 1e-3
    log("k = 1: every head's output is the selected latent row bit for bit")
