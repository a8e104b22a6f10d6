"""GPU parity of the selection variants (dsa_topk_select): a per-query k and the union with a
sliding window of recent positions, against the oracle's definition on the same score rows.

The selected index lists must be bit-identical (integers decided by float32 comparisons that both
sides make on the same values; ties to the lower position).  Rows cover short contexts (n <= k_t),
k_t = 0 (window only), clamped k_t, heavy ties, and rows longer than the LDS key cache (the
candidate path).  The selection then feeds dsa_sparse_mla with k + window index slots.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from helpers import check_mla, log
from sparse_attention_sum_amd import dsa, synth
from sparse_attention_sum_amd.device import to_device

pytestmark = pytest.mark.gpu


def _batch(q_len, max_len):
    T = len(q_len)
    dev = "cuda"
    return dsa.Batch(torch.arange(T + 1, dtype=torch.int32, device=dev), torch.arange(T, dtype=torch.int32, device=dev),
                     torch.from_numpy(np.asarray(q_len, np.int32)).to(dev), int(max_len), 1)


@pytest.mark.parametrize("k,window,max_len,ties", [
    (2048, 0, 8192, False),
    (2048, 128, 8192, True),
    (256, 512, 3000, True),
    (2048, 64, 70000, False),     # rows longer than the LDS key cache
    (64, 7, 500, True),
])
def test_topk_select_matches_oracle(k, window, max_len, ties):
    rng = np.random.default_rng(k * 7 + window + max_len)
    T = 48
    q_len = rng.integers(1, max_len + 1, T).astype(np.int32)
    q_len[:4] = [max_len, 1, min(k, max_len), 16]
    kq = rng.integers(-5, k + 50, T).astype(np.int32)
    kq[:3] = [0, k, 2 * k]
    log(f"case: topk_select k={k} window={window} max_len={max_len} ties={ties}")
    ld = (max_len + 63) // 64 * 64
    sc = rng.normal(0, 1, (T, ld)).astype(np.float32)
    if ties:
        sc = np.round(sc * 4) / 4                                      # ~30 distinct values
        sc[5, :] = 0.0
        sc[6, ::2] = -0.0
    sct = torch.from_numpy(sc).cuda()
    b = _batch(q_len, max_len)
    kqt = torch.from_numpy(kq).cuda()
    got = dsa.dsa_topk_select(sct, ld, b, k, kqt, window).cpu().numpy()
    ref = oracle.topk_select(sc.astype(np.float64), q_len, k, k_per_query=kq, window=window, nthreads=8)
    bad = [r for r in range(T) if not np.array_equal(got[r], ref[r])]
    assert not bad, f"rows {bad[:5]} differ; first: gpu {got[bad[0]][:12]} ref {ref[bad[0]][:12]}"
    # without a per-query k the union is the plain top-k plus the window
    got2 = dsa.dsa_topk_select(sct, ld, b, k, None, window).cpu().numpy()
    ref2 = oracle.topk_select(sc.astype(np.float64), q_len, k, window=window, nthreads=8)
    assert np.array_equal(got2, ref2)


def test_topk_select_plain_equals_topk():
    rng = np.random.default_rng(41)
    T, L, k = 32, 9000, 2048
    q_len = rng.integers(1, L + 1, T).astype(np.int32)
    ld = (L + 63) // 64 * 64
    sc = torch.from_numpy(rng.normal(0, 1, (T, ld)).astype(np.float32)).cuda()
    b = _batch(q_len, L)
    log("case: topk_select plain vs topk")
    a = dsa.dsa_topk_select(sc, ld, b, k, None, 0)
    c = dsa.dsa_topk(sc, ld, b, k)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_window_selection_feeds_sparse_mla():
    """decode 64 x 8192: indexer scores -> per-query k and a 256-token window -> sparse MLA over
    k + 256 slots; the output equals the oracle's attention over the same index lists."""
    spec = synth.named_spec("decode-B64-ctx8192")
    log(f"case: {spec.name} window selection -> sparse MLA")
    p = synth.build(spec)
    dp = to_device(p)
    b = dp.batch
    k, W = spec.topk, 256
    ld = dsa.score_ld(b)
    scores = dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, scale=spec.idx_scale, ld=ld)
    rng = np.random.default_rng(42)
    kq = rng.integers(0, k + 1, spec.T).astype(np.int32)
    idx = dsa.dsa_topk_select(scores, ld, b, k, torch.from_numpy(kq).cuda(), W)
    out, lse = dsa.dsa_sparse_mla(dp.q_mla, dp.latent, b, idx, spec.softmax_scale)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    rows = np.arange(0, spec.T, 8, dtype=np.int32)
    ref_idx = oracle.topk_select(scores[torch.from_numpy(rows).long().cuda()].double().cpu().numpy(), p.q_len[rows],
                                 k, k_per_query=kq[rows], window=W)
    assert np.array_equal(gi[rows], ref_idx)
    o_ref, l_ref = oracle.sparse_mla(p.q_mla, p.latent, p.q_seq, p.q_len, gi[rows], seq_stride=p.seq_stride,
                                     page_table=p.page_table, page_size=spec.page_size,
                                     softmax_scale=spec.softmax_scale, qsel=rows, nthreads=8)
    check_mla(out[torch.from_numpy(rows).long().cuda()].float().cpu().numpy(),
              lse[torch.from_numpy(rows).long().cuda()].cpu().numpy(), o_ref, l_ref, "window selection")


@pytest.mark.parametrize("max_len,k", [(131072, 2048), (100000, 2048), (70000, 1024), (80000, 4096), (40000, 2048)])
def test_two_pass_equals_one_pass(max_len, k):
    """Long rows with a workspace go through slices and a merge; the result must equal the one-pass
    selection bit for bit (ties, +-0, ragged lengths, per-query k and a window)."""
    rng = np.random.default_rng(max_len + k)
    T = 24
    q_len = rng.integers(k // 2, max_len + 1, T).astype(np.int32)
    q_len[0] = max_len
    ld = (max_len + 63) // 64 * 64
    sc = np.round(rng.normal(0, 1, (T, ld)) * 8) / 8
    sc[1, ::3] = -0.0
    sct = torch.from_numpy(sc.astype(np.float32)).cuda()
    b = _batch(q_len, max_len)
    log(f"case: two-pass top-k max_len={max_len} k={k}")
    need = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, b, k, 1)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for kq, W in ((None, 0), (torch.from_numpy(rng.integers(0, k + 1, T).astype(np.int32)).cuda(), 100)):
        one = torch.empty((T, k + W), dtype=torch.int32, device="cuda")
        two = torch.empty((T, k + W), dtype=torch.int32, device="cuda")
        bs = b.struct()
        L = dsa.load()
        assert L.dsa_topk_select(sct.data_ptr(), ld, ctypes.byref(bs), k, None if kq is None else kq.data_ptr(), W,
                                 one.data_ptr(), None, 0, None) == 0
        assert L.dsa_topk_select(sct.data_ptr(), ld, ctypes.byref(bs), k, None if kq is None else kq.data_ptr(), W,
                                 two.data_ptr(), ws.data_ptr(), need, None) == 0
        torch.cuda.synchronize()
        assert torch.equal(one, two), f"kq={kq is not None} W={W}"
    ref = oracle.topk(sc[:3], q_len[:3], k)
    got = dsa.dsa_topk(sct, ld, b, k, workspace=ws).cpu().numpy()[:3]
    for r in range(3):
        assert sorted(v for v in ref[r] if v >= 0) == [v for v in got[r] if v >= 0]


@pytest.mark.parametrize("k,window", [(2048, 0), (2048, 64), (1024, 0)])
def test_sparse_compaction_rows_match_oracle(k, window):
    """Single-pass rows of 16K-32K keys, of which at most an eighth is taken (the bitmask
    compaction), with heavy ties, +-0 and an all-equal row: the selected lists must equal the
    oracle's bit for bit (ties to the lower position, equal entries straddling 64-entry words)."""
    rng = np.random.default_rng(k + window)
    T, L = 24, 32768
    q_len = rng.integers(8 * k, L + 1, T).astype(np.int32)
    q_len[:3] = [L, 8 * k, L - 1]
    ld = L
    sc = np.round(rng.normal(0, 1, (T, ld)) * 16) / 16          # ~100 distinct values
    sc[3, :] = 1.0                                             # all equal: the first k positions
    sc[4, ::2] = -0.0
    sc[4, 1::2] = 0.0
    sc[5, : q_len[5]] = np.where(np.arange(q_len[5]) % 97 == 0, 3.0, 0.5)   # few above, many equal
    log(f"case: sparse compaction k={k} window={window}")
    sct = torch.from_numpy(sc.astype(np.float32)).cuda()
    b = _batch(q_len, L)
    got = dsa.dsa_topk_select(sct, ld, b, k, None, window).cpu().numpy()
    ref = oracle.topk_select(sc.astype(np.float32).astype(np.float64), q_len, k, window=window, nthreads=8)
    bad = [r for r in range(T) if not np.array_equal(got[r], ref[r])]
    assert not bad, f"rows {bad[:5]} differ; first: gpu {got[bad[0]][:12]} ref {ref[bad[0]][:12]}"
