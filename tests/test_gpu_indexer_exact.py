"""Exact GPU parity of the lightning indexer, and its masked entries, through every launch path.

Small-integer operands (q, k in {-3..3} stored as f32, bf16 or e4m3 codes, unit scales, weights in
{0, 1/4, 1/2, 1}, scale 1) make every score a multiple of 1/4 that binary32 holds exactly, and every
partial sum of any summation order is exact as well.  So the GPU scores must equal the oracle's bit
for bit: a dropped, doubled or mis-paired head, a wrong key row or a missing dimension all change
some score (the fp8 tolerance of 2e-2 * A would let a dropped head through).

The score buffer is filled with NaN before each call: every entry of [n_t, ld) must come back -inf
(the masked positions of the indexer-scoring step, page "一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的
四步工作流程"), so no caller ever reads stale memory past a query's context.

Launch paths (the dispatch in csrc/indexer.hip): fp8 with 32 or 64 heads and at most 8 queries per
sequence -> the fp8 decode kernel (one query per pass when max_q == 1, two otherwise); bf16 in a
contiguous cache or 64-token pages -> the DMA-streamed kernel; bf16 in 16-token pages -> the
four-query kernel; fp8 with more than 8 queries per sequence in a contiguous cache or 64-token pages
-> the fp8 streamed kernel; 1, 2, 4, 8, 16 or 32 heads in f32, and the bf16 / fp8 shapes none of the
kernels above takes (fewer than 32 heads; fp8 prefill in 16-token pages) -> the (token, head)-row MFMA
kernel (contiguous and paged, causal and ragged, tails of a 256-key chunk); f32 with 64 heads and fp8
with 48 -> the generic kernel.  The 32-head streamed
kernel (operands read from LDS a few MFMAs ahead, two workgroups per CU) has a paged and a ragged
contiguous case.
"""
import ctypes

import numpy as np
import pytest
import torch

from helpers import log, oracle_scores
from sparse_attention_sum_amd import dsa, synth
from sparse_attention_sum_amd.device import to_device

pytestmark = pytest.mark.gpu

F32, BF16, FP8 = synth.F32, synth.BF16, synth.FP8

CASES = [
    # name, ctx, nq, idx heads, dtype, paged, page size
    ("fp8-decode-1q-h64-contig", [1000, 4097, 33, 1], [1, 1, 1, 1], 64, FP8, False, 64),
    ("fp8-decode-1q-h32-paged", [1000, 4097, 33, 5], [1, 1, 1, 1], 32, FP8, True, 64),
    ("fp8-decode-2q-h64-paged", [1000, 2049, 70], [2, 2, 3], 64, FP8, True, 64),
    ("fp8-decode-2q-h32-contig", [129, 3001], [2, 2], 32, FP8, False, 64),
    ("bf16-stream-h64-contig", [300, 1025], [300, 1], 64, BF16, False, 64),
    ("bf16-stream-h32-paged64", [333, 130], [100, 130], 32, BF16, True, 64),
    ("bf16-stream-h32-contig-ragged", [1000, 77, 65], [37, 77, 9], 32, BF16, False, 64),
    ("bf16-4query-h64-page16", [333, 130], [100, 130], 64, BF16, True, 16),
    ("bf16-4query-h32-page16", [97, 40], [97, 3], 32, BF16, True, 16),
    ("f32-generic-h64", [600, 90], [3, 1], 64, F32, True, 64),
    ("f32-mfma-h8", [257, 31], [5, 31], 8, F32, False, 64),
    ("f32-mfma-h4-prefill-paged", [300, 77], [300, 5], 4, F32, True, 64),
    ("f32-mfma-h1-ragged", [100, 40, 600], [37, 40, 3], 1, F32, False, 64),
    ("f32-mfma-h2-page16", [130, 9], [65, 9], 2, F32, True, 16),
    ("f32-mfma-h16-paged", [600, 257], [9, 1], 16, F32, True, 64),
    ("f32-mfma-h32-contig", [333, 64], [33, 2], 32, F32, False, 64),
    ("bf16-rows-h16-paged", [300, 77], [300, 5], 16, BF16, True, 64),
    ("bf16-rows-h4-page16", [130, 9], [65, 9], 4, BF16, True, 16),
    ("fp8-rows-h8-decode", [1000, 4097, 33], [1, 1, 1], 8, FP8, False, 64),
    ("fp8-rows-h16-prefill-paged", [300, 130], [300, 9], 16, FP8, True, 64),
    ("fp8-rows-h32-prefill-page16", [200, 50], [200, 3], 32, FP8, True, 16),
    ("fp8-stream-12q-h64", [500, 77], [12, 2], 64, FP8, False, 64),
    ("fp8-stream-prefill-h32-paged64", [300, 130], [300, 9], 32, FP8, True, 64),
    ("fp8-generic-h48", [700, 35], [1, 1], 48, FP8, True, 64),
]


def _scores_into_nan_buffer(dp, ld):
    """dsa_indexer_scores into a NaN-filled [T, ld] buffer, through the C ABI."""
    T = dp.spec.T
    scores = torch.full((T, ld), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, dp.batch, scale=dp.spec.idx_scale,
                           scores=scores, ld=ld)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_indexer_small_integers_bit_exact_and_masked(case):
    name, ctx, nq, hi, dt, paged, ps = case
    spec = synth.Spec(name, ctx=ctx, nq=nq, idx_heads=hi, idx_dtype=dt, topk=16, mla_heads=8, paged=paged,
                      page_size=ps, seed=31)
    p = synth.small_integer_indexer(synth.build(spec), seed=7)
    dp = to_device(p)
    # an ld past max_len: the last block of each row also masks [grid end, ld)
    ld = dsa.score_ld(dp.batch) + 2048 + 3
    log(f"{name}: T={spec.T} max_len={p.max_len} ld={ld}")
    g = _scores_into_nan_buffer(dp, ld)
    ref = oracle_scores(p, ld=ld)
    for t in range(spec.T):
        n = int(p.q_len[t])
        want = ref[t, :n].astype(np.float32)
        assert np.array_equal(want.astype(np.float64), ref[t, :n]), "oracle scores not exact in binary32"
        got = g[t, :n]
        bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
        assert bad.size == 0, f"row {t}: {bad.size} scores differ, first at {bad[0]}: {got[bad[0]]} vs {want[bad[0]]}"
        tail = g[t, n:]
        assert np.all(np.isneginf(tail)), f"row {t}: {np.count_nonzero(~np.isneginf(tail))} masked entries not -inf"
    log(f"{name}: {sum(int(x) for x in p.q_len)} scores bit-exact, tails -inf")


def test_mask_through_the_c_abi_every_row_and_empty_context():
    """Called through ctypes with the C structs: a NaN-filled buffer whose rows include queries with
    no visible position (n_t = 0) and a batch with max_len = 0 (every entry masked)."""
    L = dsa.load()
    H = 64
    # batch 1: 3 queries of one sequence, n = 0, 5, 70 (fp8 decode kernel, two queries per pass)
    q_len = torch.tensor([0, 5, 70], dtype=torch.int32, device="cuda")
    q_seq = torch.zeros(3, dtype=torch.int32, device="cuda")
    cu_q = torch.tensor([0, 3], dtype=torch.int32, device="cuda")
    kdata = torch.zeros((128, 128), dtype=torch.uint8, device="cuda")
    kscale = torch.ones(128, dtype=torch.float32, device="cuda")
    q = torch.zeros((3, H, 128), dtype=torch.uint8, device="cuda")
    w = torch.ones((3, H), dtype=torch.float32, device="cuda")
    for max_len, ld in ((70, 200), (0, 96)):
        qlen = q_len if max_len else torch.zeros(3, dtype=torch.int32, device="cuda")
        b = dsa._Batch(3, 1, cu_q.data_ptr(), q_seq.data_ptr(), qlen.data_ptr(), max_len, 3)
        kc = dsa._Cache(kdata.data_ptr(), kscale.data_ptr(), dsa.DSA_FP8_E4M3, 128, 128, 128, None, 0, 64)
        scores = torch.full((3, ld), float("nan"), dtype=torch.float32, device="cuda")
        st = L.dsa_indexer_scores(ctypes.c_void_p(q.data_ptr()), dsa.DSA_FP8_E4M3, None, ctypes.c_void_p(w.data_ptr()),
                                  H, 128, ctypes.byref(kc), ctypes.byref(b), 1.0, ctypes.c_void_p(scores.data_ptr()),
                                  ld, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == dsa.DSA_OK, L.dsa_last_error()
        torch.cuda.synchronize()
        s = scores.cpu().numpy()
        n = qlen.cpu().numpy()
        for t in range(3):
            assert np.all(s[t, :n[t]] == 0.0)             # zero queries and keys score exactly 0
            assert np.all(np.isneginf(s[t, n[t]:])), f"max_len {max_len}, row {t}"
