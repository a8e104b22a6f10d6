"""Pins of the oracle's lightning indexer against closed forms, a library routine and invariants.

The definition ("一文讀懂DeepSeek-V3.2核心技術DSA", "DSA 的四步工作流程", the indexer-scoring
step; "DeepSeek 稀疏注意力路线", "两阶段流程" item 1) is
    S[t,s] = scale * sum_j w[t,j] * ReLU(q[t,j,:] . k_s),  s < n_t;  -inf for s >= n_t.
Each test below would fail for a plausible slip: ReLU after the head sum instead of per head, a
dropped head or dimension, a transposed q, a wrong sequence/page lookup, a missing scale.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _run(q, w, k, q_len, q_seq=None, **kw):
    T = q.shape[0]
    if q_seq is None:
        q_seq = np.zeros(T, dtype=np.int32)
    return oracle.indexer(q.astype(np.float32), "f32", None, w.astype(np.float32), k.astype(np.float32),
                          "f32", None, q_seq, np.asarray(q_len, dtype=np.int32), **kw)


def test_hand_example():
    """A worked example done by hand (tests/golden/indexer_hand_example.json)."""
    ex = json.load(open(os.path.join(GOLD, "indexer_hand_example.json")))
    q = np.array(ex["q"], dtype=np.float32)[None]          # [1, H, D]
    w = np.array(ex["w"], dtype=np.float32)[None]
    k = np.array(ex["k"], dtype=np.float32)
    S = _run(q, w, k, [k.shape[0]], seq_stride=k.shape[0], scale=ex["scale"])
    assert S[0].tolist() == ex["expected"]


def test_single_head_reduces_to_matmul():
    """H=1, w=1 and q,k >= 0: the ReLU is inactive and S is the plain product q k^T."""
    rng = np.random.default_rng(0)
    T, D, N = 5, 128, 70
    q = np.abs(rng.standard_normal((T, 1, D)))
    k = np.abs(rng.standard_normal((N, D)))
    w = np.ones((T, 1))
    S = _run(q, w, k, [N] * T, seq_stride=N)
    ref = np.matmul(q[:, 0, :].astype(np.float32).astype(np.float64), k.astype(np.float32).astype(np.float64).T)
    np.testing.assert_allclose(S, ref, rtol=1e-13, atol=0)


def test_unit_vector_queries_closed_form():
    """q[t,j] = e_{perm[j]}: head j's dot product is k_s[perm[j]], so
    S = scale * sum_j w_j * max(0, k_s[perm[j]]).  Sign, per-head ReLU, head/weight pairing,
    the q layout [t, head, dim] and the scale all enter."""
    rng = np.random.default_rng(1)
    H, D, N = 16, 128, 40
    perm = rng.permutation(D)[:H]
    q = np.zeros((1, H, D))
    q[0, np.arange(H), perm] = 1.0
    w = rng.uniform(0.0, 1.0, size=(1, H)).astype(np.float32)
    k = rng.integers(-4, 5, size=(N, D)).astype(np.float32)
    S = _run(q, w, k, [N], seq_stride=N, scale=0.5)
    ref = 0.5 * (np.maximum(k[:, perm], 0.0).astype(np.float64) @ w[0].astype(np.float64))
    np.testing.assert_allclose(S[0], ref, rtol=1e-15, atol=0)


def test_relu_is_per_head_not_after_sum():
    """Two heads with opposite dot products: per-head ReLU keeps the positive one; a ReLU after
    the weighted sum would give 0."""
    D = 128
    q = np.zeros((1, 2, D)); q[0, 0, 0] = 1.0; q[0, 1, 0] = -1.0
    k = np.zeros((1, D)); k[0, 0] = 3.0
    w = np.array([[1.0, 1.0]])
    S = _run(q, w, k, [1], seq_stride=1)
    assert S[0, 0] == 3.0


def test_nonnegative_with_nonnegative_weights_and_causal_mask():
    rng = np.random.default_rng(2)
    T, H, D, N = 6, 8, 128, 50
    q = rng.standard_normal((T, H, D)); k = rng.standard_normal((N, D))
    w = rng.uniform(0, 1, size=(T, H))
    q_len = np.array([1, 7, 20, 33, 49, 50], dtype=np.int32)
    S = _run(q, w, k, q_len, seq_stride=N, ld=N)
    for t in range(T):
        assert np.all(S[t, :q_len[t]] >= 0.0)
        assert np.all(np.isneginf(S[t, q_len[t]:]))
    # future rows do not influence the visible scores
    k2 = k.copy(); k2[25:] = rng.standard_normal((N - 25, D)) * 100
    S2 = _run(q, w, k2, q_len, seq_stride=N, ld=N)
    for t in range(T):
        vis = min(q_len[t], 25)
        assert np.array_equal(S[t, :vis], S2[t, :vis])


def test_zero_key_and_homogeneity_and_head_additivity():
    rng = np.random.default_rng(3)
    T, H, D, N = 3, 6, 128, 30
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    k = rng.standard_normal((N, D)).astype(np.float32)
    k[7] = 0.0
    w = rng.uniform(-1, 1, size=(T, H)).astype(np.float32)
    S = _run(q, w, k, [N] * T, seq_stride=N)
    assert np.all(S[:, 7] == 0.0)
    S2 = _run(q, w, 2.0 * k, [N] * T, seq_stride=N)                 # power of two: exact
    np.testing.assert_array_equal(S2, 2.0 * S)
    SA = _run(q[:, :2], w[:, :2], k, [N] * T, seq_stride=N)
    SB = _run(q[:, 2:], w[:, 2:], k, [N] * T, seq_stride=N)
    np.testing.assert_allclose(S, SA + SB, rtol=1e-12, atol=1e-12)
    S3 = _run(q, w, k, [N] * T, seq_stride=N, scale=3.0)
    np.testing.assert_allclose(S3, 3.0 * S, rtol=1e-15)


def test_negative_weight_gives_negative_relu():
    D = 128
    q = np.zeros((1, 1, D)); q[0, 0, 5] = 2.0
    k = np.zeros((2, D)); k[0, 5] = 1.5; k[1, 5] = -1.5
    S = _run(q, np.array([[-1.0]]), k, [2], seq_stride=2)
    assert S[0].tolist() == [-3.0, 0.0]


def _int_inputs(rng, T, H, N, D=128):
    q = rng.integers(-3, 4, size=(T, H, D)).astype(np.float32)
    k = rng.integers(-3, 4, size=(N, D)).astype(np.float32)
    w = rng.choice(np.array([0.0, 0.25, 0.5, 1.0], dtype=np.float32), size=(T, H))
    return q, k, w


def _as(x, dtype):
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_small_integers_identical_across_formats(dtype):
    """Integers in [-3, 3] are exact in f32, bf16 and e4m3; the scores must be identical."""
    rng = np.random.default_rng(4)
    T, H, N = 4, 8, 64
    q, k, w = _int_inputs(rng, T, H, N)
    q_seq = np.zeros(T, np.int32); q_len = np.array([64, 10, 33, 1], np.int32)
    ref = oracle.indexer(q, "f32", None, w, k, "f32", None, q_seq, q_len, seq_stride=N, ld=N)
    got = oracle.indexer(_as(q, dtype), dtype, None, w, _as(k, dtype), dtype, None, q_seq, q_len,
                         seq_stride=N, ld=N)
    np.testing.assert_array_equal(got, ref)


def test_fp8_scales_per_head_and_per_token():
    """q_scale[t,j] multiplies head j's product and k_scale[s] multiplies row s: with q_scale the
    indicator of one head, S equals that head alone times k_scale (positive homogeneity of ReLU)."""
    rng = np.random.default_rng(5)
    T, H, N = 2, 4, 16
    q, k, w = _int_inputs(rng, T, H, N)
    q8, k8 = _as(q, "fp8"), _as(k, "fp8")
    ks = rng.choice(np.array([0.5, 1.0, 4.0], np.float32), size=N)
    q_seq = np.zeros(T, np.int32); q_len = np.full(T, N, np.int32)
    for j in range(H):
        qs = np.zeros((T, H), np.float32); qs[:, j] = 2.0
        S = oracle.indexer(q8, "fp8", qs, w, k8, "fp8", ks, q_seq, q_len, seq_stride=N)
        Sj = oracle.indexer(q8[:, j:j + 1], "fp8", None, w[:, j:j + 1], k8, "fp8", None, q_seq, q_len,
                            seq_stride=N)
        np.testing.assert_array_equal(S, 2.0 * Sj * ks[None, :].astype(np.float64))


def test_sequences_and_pages():
    """Each query scores only its own sequence's rows, and a page-table layout of the same tokens
    gives bit-identical scores."""
    rng = np.random.default_rng(6)
    B, n, H, D, page = 3, 150, 4, 128, 64
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    w = rng.uniform(0, 1, (B, H)).astype(np.float32)
    kc = rng.standard_normal((B, n, D)).astype(np.float32)
    q_seq = np.arange(B, dtype=np.int32); q_len = np.array([150, 64, 65], np.int32)
    S = oracle.indexer(q, "f32", None, w, kc.reshape(B * n, D), "f32", None, q_seq, q_len, seq_stride=n, ld=n)
    # each sequence alone
    for b in range(B):
        Sb = oracle.indexer(q[b:b + 1], "f32", None, w[b:b + 1], kc[b], "f32", None, np.zeros(1, np.int32),
                            q_len[b:b + 1], seq_stride=n, ld=n)
        np.testing.assert_array_equal(S[b], Sb[0])
    # paged copy: 3 pages per sequence, physical pages permuted
    ppb = (n + page - 1) // page
    perm = rng.permutation(B * ppb)
    pool = np.zeros((B * ppb * page, D), np.float32)
    pt = np.zeros((B, ppb), np.int32)
    for b in range(B):
        for lp in range(ppb):
            phys = perm[b * ppb + lp]
            pt[b, lp] = phys
            rows = kc[b, lp * page:(lp + 1) * page]
            pool[phys * page:phys * page + len(rows)] = rows
    Sp = oracle.indexer(q, "f32", None, w, pool, "f32", None, q_seq, q_len, page_table=pt, page_size=page, ld=n)
    np.testing.assert_array_equal(Sp, S)


def test_query_subset_rows_match_full_run():
    rng = np.random.default_rng(7)
    T, H, D, N = 9, 4, 128, 40
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    k = rng.standard_normal((N, D)).astype(np.float32)
    w = rng.uniform(0, 1, (T, H)).astype(np.float32)
    q_len = np.arange(1, T + 1, dtype=np.int32) * 4
    q_seq = np.zeros(T, np.int32)
    S = oracle.indexer(q, "f32", None, w, k, "f32", None, q_seq, q_len, seq_stride=N, ld=N)
    sel = np.array([8, 2, 5], np.int32)
    Ss = oracle.indexer(q, "f32", None, w, k, "f32", None, q_seq, q_len, seq_stride=N, ld=N, qsel=sel)
    np.testing.assert_array_equal(Ss, S[sel])


def test_integer_inputs_expose_a_dropped_or_swapped_head():
    """Why the GPU indexer is checked bit for bit on small-integer inputs.  With q, k in {-3..3},
    unit scales and w in {0, 1/4, 1/2, 1}, every oracle score is a multiple of 1/4 that binary32
    holds exactly, so a correct kernel must reproduce it exactly.  A kernel that drops one head's term
    (its weight read as 0) or pairs two heads with each other's weights changes some of those scores,
    so the exact check fails; on N(0,1) fp8 inputs the same slips stay inside the 2e-2 * A bar."""
    from sparse_attention_sum_amd import synth
    from helpers import oracle_scores

    spec = synth.Spec("int-heads", ctx=[2000, 1500], nq=[1, 1], idx_heads=64, idx_dtype=synth.FP8, topk=64, seed=21)
    base = synth.build(spec)
    p = synth.small_integer_indexer(base, seed=3)
    S = oracle_scores(p)
    vis = np.isfinite(S)
    assert np.array_equal(S[vis].astype(np.float32).astype(np.float64), S[vis])   # exact in binary32

    def slipped(prob, j0, j1=None):
        w = prob.w.copy()
        if j1 is None:
            w[:, j0] = 0.0
        else:
            w[:, [j0, j1]] = w[:, [j1, j0]]
        import dataclasses
        return oracle_scores(dataclasses.replace(prob, w=w))

    for j in (0, 17, 63):   # every zeroed head is seen by the exact check
        if np.any(p.w[:, j] != 0):
            assert not np.array_equal(slipped(p, j)[vis], S[vis]), f"zeroed head {j} not seen"
    assert not np.array_equal(slipped(p, 5, 40)[vis], S[vis])

    # the fp8 bar on the drawn N(0,1) inputs cannot tell the slips apart from a correct result
    S_n = oracle_scores(base)
    A = oracle_scores(base, absolute=True)
    for bad in (slipped(base, 17), slipped(base, 5, 40)):
        err = np.abs(bad - S_n)[vis]
        assert np.all(err <= 2e-2 * A[vis])
