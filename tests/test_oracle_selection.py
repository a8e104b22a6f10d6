"""Pins of the oracle's selection variants: a per-query k and the union with a sliding window.

Pages: "DeepSeek-V3.2推理加速引擎深度剖析" (closing outlook: K chosen per query; the sliding-window
branch combined with the selection) and "DeepSeek-V3.2加速技术详解" (the third, sliding-window
branch).  Definition: query t takes its best k_t = clamp(kq[t], 0, k) positions (all when n_t <= k_t),
united with its last W positions, listed ascending and -1 padded to k + W.

Pins: an independent numpy implementation (lexsort + set union) on random rows with forced ties,
reduction to the pinned plain top-k when W = 0, the window-only and short-context cases, and the
size bound |result| <= k_t + W.
"""
import numpy as np

import oracle


def _brute(scores, n, kt, W, width):
    s = scores[:n]
    order = np.lexsort((np.arange(n), -s))                   # score descending, then position ascending
    chosen = set(order[:kt].tolist()) if n > kt else set(range(n))
    chosen |= set(range(max(0, n - W), n))
    out = sorted(chosen)
    return out + [-1] * (width - len(out))


def test_matches_independent_union_with_ties():
    rng = np.random.default_rng(31)
    R, L, k = 40, 300, 24
    sc = rng.integers(0, 12, (R, L)).astype(np.float64)      # many ties
    n = rng.integers(1, L + 1, R).astype(np.int32)
    kq = rng.integers(-3, k + 5, R).astype(np.int32)
    for W in (0, 1, 7, 40):
        got = oracle.topk_select(sc, n, k, k_per_query=kq, window=W)
        for r in range(R):
            kt = int(min(max(kq[r], 0), k))
            assert got[r].tolist() == _brute(sc[r], int(n[r]), kt, W, k + W), (W, r)


def test_window_zero_and_fixed_k_is_the_plain_top_k():
    rng = np.random.default_rng(32)
    R, L, k = 16, 500, 64
    sc = rng.normal(0, 1, (R, L))
    n = rng.integers(1, L + 1, R).astype(np.int32)
    got = oracle.topk_select(sc, n, k)
    ref = oracle.topk(sc, n, k)
    for r in range(R):
        assert got[r].tolist() == sorted(v for v in ref[r] if v >= 0) + [-1] * int((ref[r] < 0).sum())
    same = oracle.topk_select(sc, n, k, k_per_query=np.full(R, k, np.int32))
    assert np.array_equal(same, got)


def test_window_only_short_context_and_size_bound():
    sc = np.arange(100, dtype=np.float64)[None, :].repeat(3, 0)
    n = np.array([100, 5, 100], np.int32)
    got = oracle.topk_select(sc, n, 10, k_per_query=np.array([0, 0, 100], np.int32), window=4)
    assert got[0].tolist() == [96, 97, 98, 99] + [-1] * 10          # k_t = 0: the window alone
    assert got[1].tolist() == [1, 2, 3, 4] + [-1] * 10              # window of a 5-token context
    assert got[2].tolist() == list(range(90, 100)) + [-1] * 4       # k_t clamped to k = 10; the top-10 contain the window
    rng = np.random.default_rng(33)
    sc = rng.normal(0, 1, (30, 200))
    n = rng.integers(1, 201, 30).astype(np.int32)
    got = oracle.topk_select(sc, n, 16, window=8)
    for r in range(30):
        m = int((got[r] >= 0).sum())
        assert m <= min(int(n[r]), 24) and m >= min(int(n[r]), 16)
        assert got[r][:m].tolist() == sorted(set(got[r][:m].tolist()))
