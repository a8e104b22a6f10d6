"""GPU parity of libdsa against the CPU oracle (needs an MI355X and the built libdsa.so).

Per workload: indexer scores within rtol * A (A = the dot products' condition magnitude, computed by
the oracle on absolute values; rtol 1e-3 for f32/bf16 inputs, 2e-2 for fp8), the top-k set bit-exact
when the oracle runs on the GPU's own scores, sparse MLA on the GPU's own indices within max-abs
2e-2 / mean-abs 5e-3 / relative RMS 1e-2, and dsa_forward equal to the chained calls bit for bit.
Full-size workloads are checked on sampled query rows; small workloads on every row.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import NTHREADS, check_mla, check_scores, log, oracle_mla, oracle_scores, recall, sets
from sparse_attention_sum_amd import dsa, synth
from sparse_attention_sum_amd.device import to_device

pytestmark = pytest.mark.gpu

_current = {}


def device_problem(spec):
    key = spec.name
    if key not in _current:
        _current.clear()
        torch.cuda.empty_cache()
        log(f"building {spec.name} (T={spec.T}, B={spec.B}, max ctx={max(spec.ctx)})")
        p = synth.build(spec)
        _current[key] = to_device(p)
        torch.cuda.synchronize()
        log("uploaded")
    return _current[key]


def rtol_for(spec):
    return 2e-2 if spec.idx_dtype == synth.FP8 else 1e-3


def run_chain(dp, k):
    """indexer -> top-k -> sparse MLA through the three separate entry points."""
    b = dp.batch
    ld = dsa.score_ld(b)
    scores = dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, scale=dp.spec.idx_scale, ld=ld)
    idx = dsa.dsa_topk(scores, ld, b, k)
    out, lse = dsa.dsa_sparse_mla(dp.q_mla, dp.latent, b, idx, dp.spec.softmax_scale)
    torch.cuda.synchronize()
    return scores, idx, out, lse


def check_problem(dp, rows_idx, rows_topk, rows_mla, label):
    p, s = dp.problem, dp.spec
    k = s.topk
    scores, idx, out, lse = run_chain(dp, k)
    log(f"{label}: GPU chain done")
    # 1. indexer scores on sampled rows (rows with n <= ld only matter up to n)
    rows = np.asarray(rows_idx, dtype=np.int32)
    g = scores[torch.from_numpy(rows).long().cuda()].cpu().numpy()
    ref = oracle_scores(p, qsel=rows, ld=g.shape[1])
    A = oracle_scores(p, qsel=rows, ld=g.shape[1], absolute=True)
    worst, rel = check_scores(g, ref, A, p.q_len[rows], rtol_for(s))
    log(f"{label}: indexer ok on {len(rows)} rows, worst |err|/A = {worst:.3e}, "
        f"max |err|/|o| (|o| >= 1e-2 A) = {rel:.3e}")
    # informational: recall of the GPU selection against the oracle's own fp64 top-k
    long_rows = [r for r, t in enumerate(rows) if p.q_len[t] > k]
    if long_rows:
        want = oracle.topk(ref[long_rows], p.q_len, k, rows=rows[long_rows], nthreads=NTHREADS)
        got = idx[torch.from_numpy(rows[long_rows]).long().cuda()].cpu().numpy()
        log(f"{label}: recall of the GPU top-k vs the oracle's fp64 top-k on {len(long_rows)} rows: "
            f"{recall(got, want):.5f}")
    # 2. top-k: oracle on the GPU's own scores, bit-exact sets
    rows = np.asarray(rows_topk, dtype=np.int32)
    g = scores[torch.from_numpy(rows).long().cuda()].cpu().numpy().astype(np.float64)
    for r, t in enumerate(rows):
        g[r, p.q_len[t]:] = -np.inf
    want = oracle.topk(g, p.q_len, k, rows=rows, nthreads=NTHREADS)
    got = idx[torch.from_numpy(rows).long().cuda()].cpu().numpy()
    assert sets(got) == sets(want), f"{label}: top-k sets differ"
    for r in range(len(rows)):     # ascending positions, then -1 padding
        v = got[r][got[r] >= 0]
        assert np.all(np.diff(v) > 0) and np.all(got[r][len(v):] == -1)
    log(f"{label}: top-k bit-exact on {len(rows)} rows")
    # 3. sparse MLA on the GPU's own indices
    rows = np.asarray(rows_mla, dtype=np.int32)
    gi = idx[torch.from_numpy(rows).long().cuda()].cpu().numpy()
    o_ref, l_ref = oracle_mla(p, gi, qsel=rows)
    o_gpu = out[torch.from_numpy(rows).long().cuda()].float().cpu().numpy()
    l_gpu = lse[torch.from_numpy(rows).long().cuda()].cpu().numpy()
    mx, mean, rel = check_mla(o_gpu, l_gpu, o_ref, l_ref, label)
    log(f"{label}: sparse MLA ok on {len(rows)} rows: max-abs {mx:.2e} mean-abs {mean:.2e} rel-RMS {rel:.2e}")
    # 4. dsa_forward equals the chain bit for bit
    ind2 = torch.empty_like(idx)
    lse2 = torch.empty_like(lse)
    out2, _, _ = dsa.dsa_forward(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, k, dp.q_mla, dp.latent, dp.batch,
                                 s.softmax_scale, idx_scale=s.idx_scale, indices_out=ind2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(ind2, idx), f"{label}: forward indices differ from the chain"
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)), f"{label}: forward output differs"
    assert torch.equal(lse2, lse)
    log(f"{label}: dsa_forward == chain (bitwise)")
    return scores, idx, out


def _sample(T, q_len, k, extra=(), n=8, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(int(x) for x in extra if 0 <= x < T)
    long_rows = np.nonzero(q_len > k)[0]
    if len(long_rows):
        rows.update(int(x) for x in rng.choice(long_rows, size=min(n, len(long_rows)), replace=False))
    rows.update(int(x) for x in rng.choice(T, size=min(2, T), replace=False))
    return sorted(rows)


def test_tiny_prefill_L1024_all_rows():
    dp = device_problem(synth.named_spec("tiny-prefill-L1024"))
    T = dp.spec.T
    check_problem(dp, range(T), range(T), range(0, T, 7), "tiny prefill")


def test_tiny_prefill_L1024_peaked_softmax():
    dp = device_problem(synth.peaked_spec())
    T = dp.spec.T
    check_problem(dp, range(0, T, 97), range(T), range(0, T, 5), "peaked")


def test_decode_B64_ctx8192():
    dp = device_problem(synth.named_spec("decode-B64-ctx8192"))
    p = dp.problem
    rows = _sample(p.spec.T, p.q_len, p.spec.topk, extra=(0, 63))
    check_problem(dp, rows, range(p.spec.T), rows, "decode B64 8K")


def test_prefill_L16384_sampled():
    dp = device_problem(synth.named_spec("prefill-L16384"))
    p = dp.problem
    edge = (0, 1, 2046, 2047, 2048, 2049, 4095, 16383)
    rows = _sample(p.spec.T, p.q_len, p.spec.topk, extra=edge, n=6, seed=3)
    topk_rows = sorted(set(rows) | set(range(2040, 2060)) | set(range(16384 - 256, 16384)))
    check_problem(dp, rows, topk_rows, rows, "prefill 16K")


def test_mtp_decode_B32x2_ctx65536_paged():
    dp = device_problem(synth.named_spec("mtp-decode-B32x2-ctx65536-paged"))
    p = dp.problem
    rows = _sample(p.spec.T, p.q_len, p.spec.topk, extra=(0, 1, 62, 63), n=4, seed=4)
    check_problem(dp, rows, range(p.spec.T), rows, "MTP decode paged 64K")


def test_ragged_decode_B16_paged():
    dp = device_problem(synth.named_spec("ragged-decode-B16-paged"))
    p = dp.problem
    assert (p.q_len <= 2048).sum() >= 3
    T = p.spec.T
    check_problem(dp, range(T), range(T), range(T), "ragged decode")


# ---------------------------------------------------------------------------------------------
# small workloads that walk tile edges and every kernel path


SMALL = [
    # name, ctx, nq, idx_heads, idx dtype, k, mla heads, paged
    ("prefill-bf16-300", [300], [300], 64, synth.BF16, 64, 16, False),
    ("prefill-bf16-h32-paged", [333], [333], 32, synth.BF16, 100, 32, True),
    ("prefill-bf16-h32-contig-2seq", [700, 129], [700, 65], 32, synth.BF16, 128, 16, False),
    ("prefill-fp8-stream", [150], [150], 64, synth.FP8, 40, 128, False),
    ("prefill-fp8-stream-paged", [333, 70], [333, 70], 32, synth.FP8, 100, 16, True),
    ("decode-fp8-ragged", [1, 31, 32, 33, 64, 65, 100, 257, 1000, 2049, 4097], [1] * 11, 64, synth.FP8, 64, 128, True),
    ("mtp-fp8-h32", [70, 129, 3000], [2, 2, 2], 32, synth.FP8, 64, 64, False),
    ("decode-bf16-contig", [500, 1025], [1, 1], 64, synth.BF16, 128, 48, False),
    ("decode-f32-h8-mfma", [600, 90], [3, 1], 8, synth.F32, 50, 8, True),
    ("decode-f32-h64-generic", [600, 90], [3, 1], 64, synth.F32, 50, 8, True),
    # f32 with (token, head) MFMA rows: 16 heads, causal prefill over two sequences, 64-token pages
    ("prefill-f32-h16-paged", [333, 70], [333, 70], 16, synth.F32, 100, 16, True),
    # bf16 / fp8 with fewer than 32 indexer heads: the same (token, head)-row kernel with their MFMAs
    ("prefill-bf16-h8-rows", [333], [333], 8, synth.BF16, 100, 16, False),
    ("decode-fp8-h16-rows-paged", [600, 90, 3000], [1, 1, 1], 16, synth.FP8, 50, 8, True),
    # bf16 prefill over several sequences, queries at the end of a longer context, 64-token pages
    ("prefill-bf16-3seq-paged", [200, 777, 64], [200, 300, 64], 64, synth.BF16, 128, 16, True),
    # 16-token pages: the bf16 kernel for any cache layout
    ("prefill-bf16-page16", [333, 130], [100, 130], 64, synth.BF16, 64, 16, True, 16),
]



def test_long_rows_two_pass_topk_forward():
    """Rows longer than 32768 keys (128K, 100K, 90K, 70K and 65537, next to a 65536-key row and a
    short one): with a workspace the top-k of dsa_topk and dsa_forward runs in two passes (slices, then a
    merge of their candidates); the selected sets must still equal the oracle's on the GPU's own
    scores bit for bit, and the rest of the chain must match as for every workload."""
    spec = synth.Spec("long-rows-B6-paged", ctx=[131072, 100000, 65537, 70000, 3000, 90000], nq=[1, 1, 2, 1, 1, 1],
                      idx_dtype=synth.FP8, paged=True, seed=9)
    dp = device_problem(spec)
    assert dp.problem.max_len > 32768
    b = dp.batch
    assert dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, b, spec.topk, 1) > 0      # the two-pass path is taken
    rows = list(range(spec.T))
    check_problem(dp, rows_idx=[0, 2, 3], rows_topk=rows, rows_mla=[0, 2, 3, 5], label=spec.name)

LARGE_K = [
    # name, ctx, nq, k: k past one sparse-MLA split's 2048 slots (64 splits, the runtime combine), up to
    # the largest k the boundary takes; a row of 70000 keys selects 65536 (single-pass top-k whose
    # candidates do not fit LDS: the row is re-read from global memory on each pass), one of 30000
    # keys selects all of them
    ("largek-4096", [10000, 3000, 5000], [1, 1, 2], 4096),
    ("largek-65536", [70000, 30000], [1, 1], 65536),
]


@pytest.mark.parametrize("case", LARGE_K, ids=[c[0] for c in LARGE_K])
def test_large_k_forward(case):
    name, ctx, nq, k = case
    spec = synth.Spec(name, ctx=ctx, nq=nq, idx_dtype=synth.FP8, topk=k, mla_heads=128, paged=True, seed=17)
    dp = device_problem(spec)
    rows = list(range(spec.T))
    check_problem(dp, rows_idx=rows, rows_topk=rows, rows_mla=rows, label=spec.name)


def test_longest_context_the_boundary_takes():
    """One query over 65535 * 256 = 16776960 positions, the largest max_len the batch check accepts
    (the indexer's 256-position blocks then fill a grid dimension): the fp8 indexer over a 2.1 GB key
    cache, the single-pass top-k over a 67 MB score row (its slices would not fit LDS, so no two-pass
    split), and sparse MLA over the 2048 selected rows of a 19 GB latent cache.  Inputs are drawn on
    the device; the checks sample: the indexer on 65536 random positions against the oracle, the
    top-k set on the GPU's own scores bit for bit, the attention on the selected rows, and
    dsa_forward equal to the chain bit for bit."""
    ctx, k, scale = 65535 * 256, 2048, 1.0 / 24.0
    d = synth.build_decode_on_device(ctx, batch=1, seed=5)
    b = dsa.Batch(cu_q=d["cu_q"], q_seq=d["q_seq"], q_len=d["q_len"], max_len=ctx, max_q=1)
    kc = dsa.Cache(d["k_idx"], d["k_idx_scale"], seq_stride=ctx)
    lc = dsa.Cache(d["latent"], seq_stride=ctx)
    ld = dsa.score_ld(b)
    scores = dsa.dsa_indexer_scores(d["q_idx"], d["q_idx_scale"], d["w"], kc, b, scale=1.0, ld=ld)
    idx = dsa.dsa_topk(scores, ld, b, k)
    out, lse = dsa.dsa_sparse_mla(d["q_mla"], lc, b, idx, scale)
    torch.cuda.synchronize()
    log(f"max context {ctx}: GPU chain done")
    g = scores[0, :ctx].double().cpu().numpy()
    assert np.all(np.isneginf(scores[0, ctx:].cpu().numpy()))
    # indexer on sampled positions: the sampled key rows as one sequence of their own
    pos = np.sort(np.random.default_rng(3).choice(ctx, size=65536, replace=False)).astype(np.int64)
    kq = d["q_idx"].view(torch.uint8).cpu().numpy()
    qs, wt = d["q_idx_scale"].cpu().numpy(), d["w"].cpu().numpy()
    pos_t = torch.from_numpy(pos).cuda()
    krows = d["k_idx"][pos_t].view(torch.uint8).cpu().numpy()
    ksc = d["k_idx_scale"][pos_t].cpu().numpy()
    one = dict(q_seq=np.zeros(1, np.int32), q_len=np.array([len(pos)], np.int32), seq_stride=len(pos), nthreads=NTHREADS)
    ref = oracle.indexer(kq, "fp8", qs, wt, krows, "fp8", ksc, **one)[0, :len(pos)]
    A = oracle.indexer(kq & np.uint8(0x7F), "fp8", qs, np.abs(wt), krows & np.uint8(0x7F), "fp8", ksc, **one)[0, :len(pos)]
    err = float((np.abs(g[pos] - ref) / np.maximum(A, 1e-30)).max())
    assert err <= 2e-2, f"indexer |err|/A {err}"
    # top-k on the GPU's scores
    gi = idx[0].cpu().numpy()
    want = oracle.topk(g[None], np.array([ctx], np.int32), k, nthreads=NTHREADS)[0]
    assert sorted(gi[gi >= 0].tolist()) == sorted(want[want >= 0].tolist()), "top-k set differs"
    # attention on the selected rows
    sel = torch.from_numpy(gi.astype(np.int64)).cuda()
    lat = d["latent"][sel].view(torch.int16).cpu().numpy().view(np.uint16)
    qm = d["q_mla"].view(torch.int16).cpu().numpy().view(np.uint16)
    o_ref, l_ref = oracle.sparse_mla(qm, lat, np.zeros(1, np.int32), np.array([k], np.int32),
                                     np.arange(k, dtype=np.int32)[None], seq_stride=k, softmax_scale=scale,
                                     nthreads=NTHREADS)
    check_mla(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "max context")
    ind2 = torch.empty_like(idx)
    lse2 = torch.empty_like(lse)
    out2, _, _ = dsa.dsa_forward(d["q_idx"], d["q_idx_scale"], d["w"], kc, k, d["q_mla"], lc, b, scale,
                                 indices_out=ind2, lse=lse2)
    torch.cuda.synchronize()
    assert torch.equal(ind2, idx) and torch.equal(out2.view(torch.int16), out.view(torch.int16))
    log(f"max context {ctx}: indexer |err|/A {err:.2e} on 65536 positions, top-k exact, MLA ok, forward == chain")
    del d, scores, out, out2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_workloads_all_rows(case):
    name, ctx, nq, hi, dt, k, h, paged = case[:8]
    page_size = case[8] if len(case) > 8 else synth.PAGE
    spec = synth.Spec(name, ctx=ctx, nq=nq, idx_heads=hi, idx_dtype=dt, topk=k, mla_heads=h, paged=paged,
                      page_size=page_size, seed=11)
    dp = device_problem(spec)
    T = spec.T
    check_problem(dp, range(T), range(T), range(T), name)


def test_paged_equals_contiguous_bitwise():
    """The same tokens through a page table and through a contiguous cache give identical bits."""
    spec = synth.Spec("pg", ctx=[700, 1500], nq=[1, 2], idx_dtype=synth.FP8, topk=256, paged=True, seed=5)
    p = synth.build(spec)
    dp = to_device(p)
    # contiguous copy of the same logical rows
    B, L = spec.B, max(spec.ctx)
    rows_of = lambda b, s: p.page_table[b, s // 64] * 64 + s % 64
    lat = np.zeros((B * L, 576), np.uint16)
    kc = np.zeros((B * L, 128), np.uint8)
    ks = np.zeros(B * L, np.float32)
    for b in range(B):
        r = np.array([rows_of(b, s) for s in range(spec.ctx[b])])
        lat[b * L:b * L + len(r)] = p.latent[r]
        kc[b * L:b * L + len(r)] = p.k_idx[r]
        ks[b * L:b * L + len(r)] = p.k_idx_scale[r]
    kcache = dsa.Cache(torch.from_numpy(kc).view(torch.float8_e4m3fn).cuda(), torch.from_numpy(ks).cuda(), seq_stride=L)
    lcache = dsa.Cache(torch.from_numpy(lat).view(torch.bfloat16).cuda(), seq_stride=L)
    o1, l1, _ = dsa.dsa_forward(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, 256, dp.q_mla, dp.latent, dp.batch,
                                spec.softmax_scale, lse=torch.empty(spec.T, 128, device="cuda"))
    l2buf = torch.empty(spec.T, 128, device="cuda")
    o2, l2, _ = dsa.dsa_forward(dp.q_idx, dp.q_idx_scale, dp.w, kcache, 256, dp.q_mla, lcache, dp.batch,
                                spec.softmax_scale, lse=l2buf)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("dt,nq,hi", [(synth.BF16, [300, 1], 64), (synth.FP8, [1, 1], 64), (synth.FP8, [300, 1], 64),
                                      (synth.F32, [300, 1], 4), (synth.F32, [2, 1], 64)],
                         ids=["bf16-prefill", "fp8-decode", "fp8-prefill-stream", "f32-h4-mfma", "f32-h64-generic"])
def test_indexer_out_of_range_pages_read_as_zero_rows(dt, nq, hi):
    """Page numbers outside [0, num_pages) read as all-zero key rows: those tokens score exactly 0
    (ReLU(0) = 0) and every other score is unchanged, bit for bit."""
    spec = synth.Spec(f"badpage-{dt}-{nq[0]}-h{hi}", ctx=[700, 300], nq=nq, idx_heads=hi, idx_dtype=dt, topk=64,
                      paged=True, seed=13)
    p = synth.build(spec)
    dp = to_device(p)
    b = dp.batch
    ld = dsa.score_ld(b)
    s1 = dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, scale=spec.idx_scale, ld=ld)
    pt = p.page_table.copy()
    num_pages = p.k_idx.shape[0] // synth.PAGE
    pt[0, 2] = -1                      # tokens 128..191 of sequence 0
    pt[0, 5] = num_pages               # tokens 320..383
    pt[1, 1] = -7                      # tokens 64..127 of sequence 1
    kc = dsa.Cache(dp.k_cache.data, dp.k_cache.scale, page_table=torch.from_numpy(pt).cuda(), page_size=synth.PAGE)
    s2 = dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, kc, b, scale=spec.idx_scale, ld=ld)
    torch.cuda.synchronize()
    s1, s2 = s1.cpu().numpy(), s2.cpu().numpy()
    bad = {0: [(128, 192), (320, 384)], 1: [(64, 128)]}
    for t in range(spec.T):
        n = int(p.q_len[t])
        seq = int(p.q_seq[t])
        mask = np.zeros(n, bool)
        for lo, hi in bad[seq]:
            mask[lo:min(hi, n)] = True
        assert np.all(s2[t, :n][mask] == 0.0), f"row {t}: a token of a bad page scored nonzero"
        assert np.array_equal(s2[t, :n][~mask], s1[t, :n][~mask]), f"row {t}: other scores changed"


def test_deterministic_repeat():
    spec = synth.named_spec("ragged-decode-B16-paged")
    dp = device_problem(spec)
    a = run_chain(dp, spec.topk)
    b = run_chain(dp, spec.topk)
    for x, y in zip(a, b):
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y)


def test_topk_stress_rows():
    """Ties, signed zeros, constant rows, monotone rows, rows longer than the LDS cache."""
    rng = np.random.default_rng(9)
    rows, lens = [], []
    L = 40000
    def add(v):
        row = np.full(L, np.nan, np.float32)
        row[:len(v)] = v
        rows.append(row); lens.append(len(v))
    add(np.zeros(5000, np.float32))                                        # all equal
    add(np.where(rng.random(6000) < 0.5, 0.0, -0.0).astype(np.float32))    # +0 / -0 mix
    add(np.arange(7000, dtype=np.float32))                                 # monotone
    add(-np.arange(7000, dtype=np.float32))
    add(rng.integers(0, 5, 9000).astype(np.float32))                       # heavy ties
    add(rng.standard_normal(L).astype(np.float32))                         # longer than LDS cache
    add(np.concatenate([np.full(3000, 1e30), np.full(3000, -1e30)]).astype(np.float32))
    add(rng.standard_normal(100).astype(np.float32))                       # n <= k
    v = rng.standard_normal(5000).astype(np.float32); v[::2] = -np.inf     # -inf entries
    add(v)
    add(np.concatenate([np.full(100, 3.0), np.full(4000, 2.0)]).astype(np.float32))  # threshold inside a tie run
    # rows longer than the LDS key cache: candidates gathered into LDS (integer ties at the
    # threshold), and a tie run at the threshold larger than the candidate area (global fallback)
    add(rng.integers(0, 100, 36000).astype(np.float32))
    add(np.concatenate([np.full(20000, 0.5), np.full(20000, 1.0)]).astype(np.float32)[rng.permutation(40000)])
    S = np.stack(rows)
    q_len = np.array(lens, np.int32)
    T = len(lens)
    for k in (1, 37, 2048, 4096):
        batch = dsa.Batch(cu_q=torch.tensor([0, T], dtype=torch.int32, device="cuda"),
                          q_seq=torch.zeros(T, dtype=torch.int32, device="cuda"),
                          q_len=torch.from_numpy(q_len).cuda(), max_len=L, max_q=T)
        idx = dsa.dsa_topk(torch.from_numpy(S).cuda(), L, batch, k)
        torch.cuda.synchronize()
        S64 = S.astype(np.float64)
        for r in range(T):
            S64[r, q_len[r]:] = -np.inf
        want = oracle.topk(S64, q_len, k)
        assert sets(idx.cpu().numpy()) == sets(want), f"k={k}"


def test_sparse_mla_user_indices_and_edge_cases():
    """Unsorted indices, -1 in the middle, out-of-range entries, no valid entry, k not a multiple
    of the tile, several head counts."""
    rng = np.random.default_rng(10)
    for H in (8, 16, 48, 128):
        spec = synth.Spec(f"mla-H{H}", ctx=[300, 80, 5000], nq=[1, 1, 1], idx_dtype=synth.FP8, topk=100,
                          mla_heads=H, seed=H)
        p = synth.build(spec)
        dp = to_device(p)
        k = 100
        idx = np.full((3, k), -1, np.int32)
        idx[0, :70] = rng.permutation(300)[:70]
        idx[0, 10] = -1; idx[0, 20] = 300; idx[0, 30] = 10 ** 6          # skipped entries
        idx[1, :] = -1                                                    # nothing selected
        idx[2, :] = rng.choice(5000, size=k, replace=False)
        it = torch.from_numpy(idx).cuda()
        out, lse = dsa.dsa_sparse_mla(dp.q_mla, dp.latent, dp.batch, it, spec.softmax_scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle_mla(p, idx)
        check_mla(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"H={H}")
        assert torch.all(out[1] == 0) and torch.all(torch.isneginf(lse[1]))


def test_sparse_mla_logits_far_above_the_first_tile():
    """A selected row whose logit is up to ~190 nats above every logit of the first tile: the running
    sum against the first tile's reference overflows the 2^64 margin, so the kernel must take its
    exact two-pass path.  Head h's query is 2 c_h in every dim, c_h spread over [0.05, 2] (each head
    its own query and its own mix of the large row and the others), and that row is 2 in every dim
    (exact in bf16): its logit is 576 * 4 c_h / 24 = 96 c_h."""
    import torch as _t
    rng = np.random.default_rng(12)
    for H in (16, 128):
        spec = synth.Spec(f"mla-far-H{H}", ctx=[300, 300], nq=[1, 1], idx_dtype=synth.FP8, topk=100,
                          mla_heads=H, seed=H + 1)
        p = synth.build(spec)
        bits2 = np.uint16(0x4000)                                  # bf16 2.0
        c = np.linspace(0.05, 2.0, H).astype(np.float32)
        qh = _t.from_numpy(2.0 * c).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16)
        p.q_mla[:] = qh[None, :, None]
        big = 1 * p.seq_stride + 250                               # sequence 1, position 250
        p.latent[big] = bits2
        dp = to_device(p)
        k = 100
        idx = np.full((2, k), -1, np.int32)
        idx[0, :80] = rng.permutation(240)[:80]                    # no large row: the fast path
        idx[1, :79] = rng.permutation(240)[:79]
        idx[1, 79] = 250                                           # the large row, in the third tile
        it = torch.from_numpy(idx).cuda()
        out, lse = dsa.dsa_sparse_mla(dp.q_mla, dp.latent, dp.batch, it, spec.softmax_scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle_mla(p, idx)
        check_mla(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, f"far H={H}")
        # where the large row's logit is far above the rest it dominates: the output is its values
        dom = c >= 0.5
        assert np.abs(out[1, torch.from_numpy(np.nonzero(dom)[0]).cuda()].float().cpu().numpy() - 2.0).max() < 1e-2
        assert np.abs(o_ref[1] - o_ref[1].mean(axis=0)).max() > 0.1      # the heads differ


def test_empty_batch_is_a_no_op():
    T = 0
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    batch = dsa.Batch(cu_q=torch.zeros(2, dtype=torch.int32, device="cuda"), q_seq=z, q_len=z, max_len=0, max_q=1)
    lat = dsa.Cache(torch.zeros(64, 576, dtype=torch.bfloat16, device="cuda"), seq_stride=64)
    out, lse = dsa.dsa_sparse_mla(torch.zeros(0, 8, 576, dtype=torch.bfloat16, device="cuda"), lat, batch,
                                  torch.zeros(0, 16, dtype=torch.int32, device="cuda"), 1 / 24)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 512)
