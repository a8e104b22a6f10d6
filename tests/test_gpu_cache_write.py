"""GPU parity of the cache write path (dsa_cache_append, dsa_rope_queries) against the CPU oracle.

Both sides rotate in double and round once to binary32, then store (bf16 round to nearest even,
e4m3 with one scale per 128-wide row).  Stored codes must be bit-identical, except where the
rounding decision sits on a tie: the two sides' double-precision cos / sin / pow may differ in the
last bit, which can move a binary32 value by one ulp.  Such a code may differ by one step, and only
where the oracle's value lies within a few binary32 ulps of the midpoint between the two codes, plus
the absolute error the angle can carry: one ulp of base^(-2i/d) from the two math libraries is an
angle error of about 2^-52 * position, i.e. an error of up to 1e-15 * (position + 1) times the
row's largest value (at position 131071 and angles near 1e5 rad this is several binary32 ulps of a
small rotated value).
fp8 row scales must agree to one binary32 ulp (the row maximum can move by one ulp the same way).
Rows outside the call's tokens must be untouched, and tokens with no slot are not written.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from helpers import check_mla, log
from sparse_attention_sum_amd import dsa

pytestmark = pytest.mark.gpu

SENT8 = 0x5a            # sentinel byte of unwritten fp8 rows
SENT16 = 0x1234         # sentinel of unwritten bf16 rows


def bits16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _ulp32(v):
    v = np.abs(v.astype(np.float32))
    return (np.nextafter(v, np.float32(np.inf)) - v).astype(np.float64)


def angle_tol(val, pos_rows):
    """Per element of val [rows, width]: 1e-15 * (position + 1) * the row's largest |value|."""
    v = np.abs(val.astype(np.float64))
    m = v.max(axis=-1, keepdims=True) * 1e-15 * (np.abs(np.asarray(pos_rows, np.float64))[:, None] + 1.0)
    return np.broadcast_to(m, v.shape).ravel()


def check_bf16(gpu, ref, val, atol, label):
    """gpu / ref: bf16 bits; val: the oracle's binary32 values before rounding, [rows, width];
    atol: per-element absolute tolerance of val (angle_tol)."""
    gpu, ref, val = gpu.ravel(), ref.ravel(), val.ravel().astype(np.float32)
    bad = gpu != ref
    if bad.any():
        g, r, v = gpu[bad].astype(np.int64), ref[bad].astype(np.int64), val[bad]
        assert np.all(np.abs(g - r) == 1), f"{label}: bf16 codes more than one step apart"
        lo = np.minimum(g, r).astype(np.uint32) << 16
        mid = (lo.view(np.float32).astype(np.float64) + (lo + 0x10000).view(np.float32).astype(np.float64)) / 2
        tol = 4 * _ulp32(v) + atol[bad]
        assert np.all(np.abs(np.abs(v.astype(np.float64)) - np.abs(mid)) <= tol), f"{label}: bf16 off a tie"
        assert bad.mean() < 1e-3, f"{label}: {bad.sum()} bf16 ties"
    log(f"{label}: bf16 {gpu.size} values, {int(bad.sum())} at ties")


def check_fp8(gpu, gscale, ref, rscale, val, atol, label):
    """gpu / ref: e4m3 codes [rows, 128]; scales [rows]; val: the oracle's binary32 values; atol as
    for check_bf16."""
    np.testing.assert_allclose(gscale, rscale, rtol=2.5e-7, atol=0, err_msg=f"{label}: fp8 scales")
    bad = gpu != ref
    if bad.any():
        rows = np.nonzero(bad)[0]
        g = oracle.decode(gpu[bad], "fp8"); r = oracle.decode(ref[bad], "fp8")
        x = val[bad].astype(np.float64) / rscale[rows].astype(np.float64)
        assert np.all(np.sign(g) * np.sign(r) >= 0), f"{label}: fp8 sign"
        # adjacent codes, and x within a few ulps (relative) of their midpoint
        assert np.all(np.abs(gpu[bad].astype(np.int64) - ref[bad].astype(np.int64)) == 1), f"{label}: fp8 codes apart"
        tol = 1e-5 * np.abs(x) + 1e-9 + atol.reshape(gpu.shape)[bad] / rscale[rows]
        assert np.all(np.abs(np.abs(x) - np.abs(g + r) / 2) <= tol), f"{label}: fp8 off a tie"
        assert bad.mean() < 1e-3, f"{label}: {bad.sum()} fp8 ties"
    log(f"{label}: fp8 {gpu.size} codes, {int(bad.sum())} at ties")


def _tokens(rng, B, S, T):
    seq = rng.integers(0, B, 4 * T).astype(np.int32)
    pos = rng.integers(0, S, 4 * T).astype(np.int32)
    _, first = np.unique(np.stack([seq, pos], 1), axis=0, return_index=True)
    keep = np.sort(first)[:T]
    return seq[keep], pos[keep]


def _rope_t(r):
    return None if r is None else (r.offset, r.dim, 1 if r.interleaved else 0, float(r.base))


def _rows_of(seq, pos, S=None, pt=None, ps=64):
    if pt is None:
        return seq.astype(np.int64) * S + pos
    return pt[seq, pos // ps].astype(np.int64) * ps + pos % ps


@pytest.mark.parametrize("layout,kdt,ksrc,kr,lr", [
    ("contiguous", "fp8", "f32", dsa.Rope(0, 64, True, 10000.0), dsa.Rope(512, 64, True, 10000.0)),
    ("paged", "bf16", "bf16", dsa.Rope(64, 64, False, 50000.0), dsa.Rope(512, 64, False, 10000.0)),
    ("paged", "fp8", "bf16", dsa.Rope(0, 128, True, 10000.0), dsa.Rope(448, 128, True, 1e6)),
    ("contiguous", "f32", "f32", None, None),
])
def test_cache_append_matches_oracle(layout, kdt, ksrc, kr, lr):
    rng = np.random.default_rng(zlib.crc32(f"{layout}/{kdt}/{ksrc}/{kr}".encode()))
    B, S, ps = 3, 8192, 64
    T = 700
    seq, pos = _tokens(rng, B, S, T)
    T = len(seq)
    log(f"case: cache_append {layout} k={kdt} src={ksrc} T={T}")
    kx = rng.normal(0, 1, (T, 128)).astype(np.float32)
    lx = (rng.normal(0, 1, (T, 576)) / 24).astype(np.float32)
    kt = torch.from_numpy(kx).cuda()
    if ksrc == "bf16":
        kt = kt.to(torch.bfloat16)
        kx_src = bits16(kt)
    else:
        kx_src = kx
    lt = torch.from_numpy(lx).cuda().to(torch.bfloat16)
    lx_src = bits16(lt)
    rows = B * S
    pt = None
    if layout == "paged":
        pt = rng.permutation(rows // ps).astype(np.int32).reshape(B, S // ps)
    # GPU caches, filled with sentinels
    kdtype = {"fp8": torch.uint8, "bf16": torch.int16, "f32": torch.float32}[kdt]
    kc = torch.full((rows, 128), SENT8 if kdt == "fp8" else (SENT16 if kdt == "bf16" else 7.0), dtype=kdtype, device="cuda")
    ks = torch.full((rows,), -1.0, dtype=torch.float32, device="cuda") if kdt == "fp8" else None
    lc = torch.full((rows, 576), SENT16, dtype=torch.int16, device="cuda")
    ptt = None if pt is None else torch.from_numpy(pt).cuda()
    kcache = dsa.Cache(kc, ks, seq_stride=S, page_table=ptt, page_size=ps,
                       dtype={"fp8": dsa.DSA_FP8_E4M3, "bf16": dsa.DSA_BF16, "f32": dsa.DSA_F32}[kdt])
    lcache = dsa.Cache(lc, None, seq_stride=S, page_table=ptt, page_size=ps, dtype=dsa.DSA_BF16)
    dsa.dsa_cache_append(kt, lt, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), B, kcache, lcache,
                         kr, lr)
    torch.cuda.synchronize()
    r = _rows_of(seq, pos, S, pt, ps)
    # oracle values of the written rows
    kval = oracle.rope_rows(kx_src, ksrc, pos, _rope_t(kr))
    lval = oracle.rope_rows(lx_src, "bf16", pos, _rope_t(lr))
    kst, ksc = oracle.rope_store(kx_src[:, None, :], ksrc, pos, _rope_t(kr), kdt)
    lst, _ = oracle.rope_store(lx_src[:, None, :], "bf16", pos, _rope_t(lr), "bf16")
    gk = kc.cpu().numpy()
    gl = lc.cpu().numpy().view(np.uint16)
    if kdt == "fp8":
        check_fp8(gk[r], ks.cpu().numpy()[r], kst[:, 0], ksc[:, 0], kval, angle_tol(kval, pos), f"{layout} k cache")
    elif kdt == "bf16":
        check_bf16(gk.view(np.uint16)[r], kst[:, 0], kval, angle_tol(kval, pos), f"{layout} k cache")
    else:
        assert np.array_equal(gk[r], kst[:, 0])                   # no rotation: an exact copy
    check_bf16(gl[r], lst[:, 0], lval, angle_tol(lval, pos), f"{layout} latent")
    # every other row untouched
    other = np.ones(rows, bool); other[r] = False
    if kdt == "fp8":
        assert np.all(gk[other] == SENT8) and np.all(ks.cpu().numpy()[other] == -1.0)
    elif kdt == "bf16":
        assert np.all(gk.view(np.uint16)[other] == SENT16)
    else:
        assert np.all(gk[other] == 7.0)
    assert np.all(gl[other] == SENT16)


def test_cache_append_skips_tokens_without_a_slot():
    rng = np.random.default_rng(5)
    B, S, ps = 2, 256, 64
    pt = rng.permutation(B * S // ps).astype(np.int32).reshape(B, S // ps)
    pt[1, 1] = -1
    pt[0, 3] = 10_000                                    # a page past the cache
    seq = np.array([2, -1, 0, 0, 1, 0, 1], np.int32)
    pos = np.array([0, 5, -1, S, 64 + 5, 3 * 64 + 1, 7], np.int32)   # only the last token has a slot
    log("case: cache_append tokens without a slot")
    kc = torch.full((B * S, 128), SENT8, dtype=torch.uint8, device="cuda")
    ks = torch.full((B * S,), -1.0, device="cuda")
    lc = torch.full((B * S, 576), SENT16, dtype=torch.int16, device="cuda")
    ptt = torch.from_numpy(pt).cuda()
    kx = torch.randn(7, 128, device="cuda")
    lx = torch.randn(7, 576, device="cuda").to(torch.bfloat16)
    dsa.dsa_cache_append(kx, lx, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), B,
                         dsa.Cache(kc, ks, page_table=ptt, page_size=ps, dtype=dsa.DSA_FP8_E4M3),
                         dsa.Cache(lc, None, page_table=ptt, page_size=ps, dtype=dsa.DSA_BF16),
                         dsa.Rope(0, 64), dsa.Rope(512, 64))
    torch.cuda.synchronize()
    row = int(pt[1, 0]) * ps + 7
    gk, gl = kc.cpu().numpy(), lc.cpu().numpy()
    written_k = np.nonzero(np.any(gk != SENT8, axis=1))[0]
    written_l = np.nonzero(np.any(gl != SENT16, axis=1))[0]
    assert written_k.tolist() == [row] and written_l.tolist() == [row]


@pytest.mark.parametrize("qsrc,qdst,ri,rm", [
    ("f32", "fp8", dsa.Rope(0, 64, True, 10000.0), dsa.Rope(512, 64, True, 10000.0)),      # 16-byte path, adjacent pairs
    ("bf16", "bf16", dsa.Rope(64, 64, False, 10000.0), dsa.Rope(512, 64, False, 10000.0)), # 16-byte path, halves
    ("f32", "f32", dsa.Rope(2, 126, True, 500.0), dsa.Rope(510, 66, True, 10000.0)),      # 2-byte path (unaligned span)
    ("bf16", "fp8", dsa.Rope(0, 128, False, 1e6), dsa.Rope(0, 576, False, 10000.0)),      # whole rows rotated
])
def test_rope_queries_matches_oracle(qsrc, qdst, ri, rm):
    rng = np.random.default_rng(zlib.crc32(f"{qsrc}/{qdst}/{ri}/{rm}".encode()))
    T, HI, H = 48, 64, 128
    log(f"case: rope_queries {qsrc} -> {qdst}")
    pos = rng.integers(0, 131072, T).astype(np.int32)
    qi = rng.normal(0, 1, (T, HI, 128)).astype(np.float32)
    qit = torch.from_numpy(qi).cuda()
    if qsrc == "bf16":
        qit = qit.to(torch.bfloat16)
        qi_src = bits16(qit)
    else:
        qi_src = qi
    qm = torch.from_numpy((rng.normal(0, 1, (T, H, 576)) / 24).astype(np.float32)).cuda().to(torch.bfloat16)
    qm_before = bits16(qm).copy()
    odt = {"fp8": torch.uint8, "bf16": torch.int16, "f32": torch.float32}[qdst]
    qo = torch.zeros((T, HI, 128), dtype=odt, device="cuda")
    qs = torch.zeros((T, HI), device="cuda") if qdst == "fp8" else None
    # the binding picks the output code from the tensor's dtype: uint8 -> fp8, int16 -> bf16
    dsa.dsa_rope_queries(qit, qo, qs, qm, torch.from_numpy(pos).cuda(), ri, rm)
    torch.cuda.synchronize()
    val = oracle.rope_rows(qi_src.reshape(T * HI, 128), qsrc, np.repeat(pos, HI), _rope_t(ri))
    vtol = angle_tol(val, np.repeat(pos, HI))
    ref, rsc = oracle.rope_store(qi_src, qsrc, pos, _rope_t(ri), qdst)
    if qdst == "fp8":
        check_fp8(qo.cpu().numpy().reshape(T * HI, 128), qs.cpu().numpy().ravel(), ref.reshape(T * HI, 128),
                  rsc.ravel(), val, vtol, "indexer q")
    elif qdst == "bf16":
        check_bf16(bits16(qo), ref, val, vtol, "indexer q")
    else:
        got = qo.cpu().numpy().reshape(T * HI, 128).astype(np.float64)
        r64 = ref.reshape(T * HI, 128)
        tol = _ulp32(r64) + vtol.reshape(T * HI, 128)
        assert np.all(np.abs(got - r64.astype(np.float64)) <= tol)
    g = bits16(qm)
    span = np.zeros(576, bool); span[rm.offset:rm.offset + rm.dim] = True
    assert np.array_equal(g[..., ~span], qm_before[..., ~span])   # outside the span: untouched
    mval = oracle.rope_rows(qm_before.reshape(T * H, 576), "bf16", np.repeat(pos, H), _rope_t(rm))
    mref, _ = oracle.rope_store(qm_before, "bf16", pos, _rope_t(rm), "bf16")
    check_bf16(g.reshape(T * H, 576)[:, span], mref.reshape(T * H, 576)[:, span], mval[:, span],
               angle_tol(mval[:, span], np.repeat(pos, H)), "mla q")


def test_write_path_then_forward():
    """A decode step built by the write path: every token of 4 sequences appended (fp8 indexer keys,
    bf16 latent, paged), the queries rotated (indexer q to fp8), then dsa_forward; the forward's
    output equals the oracle's forward on the caches and queries the GPU wrote."""
    rng = np.random.default_rng(21)
    B, ctx, ps, HI, H, k = 4, 3000, 64, 64, 128, 2048
    S = (ctx + ps - 1) // ps * ps
    log("case: write path -> dsa_forward, 4 x 3000 paged")
    npages = B * S // ps
    pt = rng.permutation(npages).astype(np.int32).reshape(B, S // ps)
    ptt = torch.from_numpy(pt).cuda()
    seq = np.repeat(np.arange(B, dtype=np.int32), ctx)
    pos = np.tile(np.arange(ctx, dtype=np.int32), B)
    kx = torch.randn(B * ctx, 128, device="cuda")
    lx = (torch.randn(B * ctx, 576, device="cuda") / 24).to(torch.bfloat16)
    kc = torch.zeros((npages * ps, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((npages * ps,), device="cuda")
    lc = torch.zeros((npages * ps, 576), dtype=torch.int16, device="cuda")
    kcache = dsa.Cache(kc, ks, page_table=ptt, page_size=ps, dtype=dsa.DSA_FP8_E4M3)
    lcache = dsa.Cache(lc, None, page_table=ptt, page_size=ps, dtype=dsa.DSA_BF16)
    kr, lr = dsa.Rope(0, 64), dsa.Rope(512, 64)
    dsa.dsa_cache_append(kx, lx, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), B, kcache, lcache, kr, lr)
    # one query per sequence at the last position
    qpos = np.full(B, ctx - 1, np.int32)
    qi = torch.randn(B, HI, 128, device="cuda")
    q8 = torch.zeros((B, HI, 128), dtype=torch.uint8, device="cuda")
    qsc = torch.zeros((B, HI), device="cuda")
    qm = (torch.randn(B, H, 576, device="cuda") / 24).to(torch.bfloat16)
    dsa.dsa_rope_queries(qi, q8, qsc, qm, torch.from_numpy(qpos).cuda(), kr, lr)
    w = torch.rand(B, HI, device="cuda")
    cu = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    qseq = torch.arange(B, dtype=torch.int32, device="cuda")
    qlen = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    batch = dsa.Batch(cu, qseq, qlen, ctx, 1)
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out, lse, _ = dsa.dsa_forward(q8, qsc, w, kcache, k, qm, lcache, batch, 1.0 / 24.0,
                                  indices_out=idx, lse=torch.empty((B, H), device="cuda"))
    torch.cuda.synchronize()
    # oracle forward on the GPU-written caches and queries
    kw = dict(page_table=pt, page_size=ps)
    sc = oracle.indexer(q8.cpu().numpy(), "fp8", qsc.cpu().numpy(), w.cpu().numpy(), kc.cpu().numpy(), "fp8",
                        ks.cpu().numpy(), qseq.cpu().numpy(), qlen.cpu().numpy(), **kw)
    # the top-k set on the GPU's scores is checked elsewhere; here the selection is the oracle's on its
    # own scores, compared as sets
    ref_idx = oracle.topk(sc, qlen.cpu().numpy(), k)
    gi = idx.cpu().numpy()
    for t in range(B):
        common = len(set(gi[t].tolist()) & set(ref_idx[t].tolist()))
        assert common >= k - 8, f"query {t}: {k - common} selections differ"   # fp8 score ties / near-ties only
    o_ref, l_ref = oracle.sparse_mla(bits16(qm), lc.cpu().numpy().view(np.uint16), qseq.cpu().numpy(),
                                     qlen.cpu().numpy(), gi, softmax_scale=1.0 / 24.0, **kw)
    check_mla(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "write path forward")


def test_prefill_size_write_path_sampled():
    """Full prefill size (16384 tokens, 64 indexer heads, 128 MLA heads) on sampled tokens."""
    rng = np.random.default_rng(22)
    T, HI, H, ps = 16384, 64, 128, 64
    log("case: write path at 16384 tokens")
    pos = np.arange(T, dtype=np.int32); seq = np.zeros(T, np.int32)
    pt = rng.permutation(T // ps).astype(np.int32).reshape(1, T // ps)
    ptt = torch.from_numpy(pt).cuda()
    kx = torch.randn(T, 128, device="cuda").to(torch.bfloat16)
    lx = (torch.randn(T, 576, device="cuda") / 24).to(torch.bfloat16)
    kc = torch.zeros((T, 128), dtype=torch.uint8, device="cuda"); ks = torch.zeros(T, device="cuda")
    lc = torch.zeros((T, 576), dtype=torch.int16, device="cuda")
    kr, lr = dsa.Rope(0, 64), dsa.Rope(512, 64)
    dsa.dsa_cache_append(kx, lx, torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(), 1,
                         dsa.Cache(kc, ks, page_table=ptt, page_size=ps, dtype=dsa.DSA_FP8_E4M3),
                         dsa.Cache(lc, None, page_table=ptt, page_size=ps, dtype=dsa.DSA_BF16), kr, lr)
    qi = torch.randn(T, HI, 128, device="cuda").to(torch.bfloat16)
    q8 = torch.zeros((T, HI, 128), dtype=torch.uint8, device="cuda"); qs = torch.zeros((T, HI), device="cuda")
    qm = (torch.randn(T, H, 576, device="cuda") / 24).to(torch.bfloat16)
    samp = np.sort(rng.choice(T, 96, replace=False)).astype(np.int64)
    samp_t = torch.from_numpy(samp).cuda()
    qm_before = bits16(qm[samp_t])
    dsa.dsa_rope_queries(qi, q8, qs, qm, torch.from_numpy(pos).cuda(), kr, lr)
    torch.cuda.synchronize()
    r = pt[0, samp // ps].astype(np.int64) * ps + samp % ps
    kx_s = bits16(kx)[samp]; lx_s = bits16(lx)[samp]
    kst, ksc = oracle.rope_store(kx_s[:, None], "bf16", pos[samp], _rope_t(kr), "fp8")
    kv = oracle.rope_rows(kx_s, "bf16", pos[samp], _rope_t(kr))
    check_fp8(kc.cpu().numpy()[r], ks.cpu().numpy()[r], kst[:, 0], ksc[:, 0], kv, angle_tol(kv, pos[samp]),
              "prefill k cache")
    lst, _ = oracle.rope_store(lx_s[:, None], "bf16", pos[samp], _rope_t(lr), "bf16")
    lv = oracle.rope_rows(lx_s, "bf16", pos[samp], _rope_t(lr))
    check_bf16(lc.cpu().numpy().view(np.uint16)[r], lst[:, 0], lv, angle_tol(lv, pos[samp]), "prefill latent")
    qi_s = bits16(qi[samp_t])
    qref, qsref = oracle.rope_store(qi_s, "bf16", pos[samp], _rope_t(kr), "fp8")
    qval = oracle.rope_rows(qi_s.reshape(-1, 128), "bf16", np.repeat(pos[samp], HI), _rope_t(kr))
    check_fp8(q8[samp_t].cpu().numpy().reshape(-1, 128), qs[samp_t].cpu().numpy().ravel(), qref.reshape(-1, 128),
              qsref.ravel(), qval, angle_tol(qval, np.repeat(pos[samp], HI)), "prefill indexer q")
    mref, _ = oracle.rope_store(qm_before, "bf16", pos[samp], _rope_t(lr), "bf16")
    mval = oracle.rope_rows(qm_before.reshape(-1, 576), "bf16", np.repeat(pos[samp], H), _rope_t(lr))
    check_bf16(bits16(qm[samp_t]).reshape(-1, 576), mref.reshape(-1, 576), mval,
               angle_tol(mval, np.repeat(pos[samp], H)), "prefill mla q")
