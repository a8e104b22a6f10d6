"""Shared helpers for the GPU parity tests: oracle calls on a synth.Problem, tolerance checks."""
import os
import sys
import time

import numpy as np

import oracle

NTHREADS = min(16, len(os.sched_getaffinity(0)))


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


def cache_kw(p):
    return dict(seq_stride=p.seq_stride, page_table=p.page_table, page_size=p.spec.page_size)


def oracle_scores(p, qsel=None, ld=None, absolute=False):
    """Oracle indexer scores for query rows qsel; absolute=True gives the condition magnitude
    A = |scale| sum_j |w'_j| sum_i |q_ji k_i| (the oracle run on absolute values)."""
    s = p.spec
    q, k, w = p.q_idx, p.k_idx, p.w
    if absolute:
        if s.idx_dtype == "f32":
            q, k = np.abs(q), np.abs(k)
        elif s.idx_dtype == "bf16":
            q, k = q & np.uint16(0x7FFF), k & np.uint16(0x7FFF)
        else:
            q, k = q & np.uint8(0x7F), k & np.uint8(0x7F)
        w = np.abs(w)
    return oracle.indexer(q, s.idx_dtype, p.q_idx_scale, w, k, s.idx_dtype, p.k_idx_scale, p.q_seq, p.q_len,
                          scale=abs(s.idx_scale) if absolute else s.idx_scale, ld=ld, qsel=qsel,
                          nthreads=NTHREADS, **cache_kw(p))


def oracle_mla(p, idx, qsel=None):
    s = p.spec
    return oracle.sparse_mla(p.q_mla, p.latent, p.q_seq, p.q_len, idx, softmax_scale=s.softmax_scale,
                             qsel=qsel, nthreads=NTHREADS, **cache_kw(p))


def check_scores(gpu, ref, A, q_len_rows, rtol):
    """|g - o| <= rtol * A on every visible entry (A: the dot products' condition magnitude).
    Returns (max |g - o| / A, max |g - o| / |o| over the entries with |o| >= 1e-2 A); the second is
    the relative error reported beside the bar, on the scores that are not cancellations."""
    worst = rel = 0.0
    for r in range(gpu.shape[0]):
        n = int(q_len_rows[r])
        g = gpu[r, :n].astype(np.float64)
        o = ref[r, :n]
        a = A[r, :n]
        err = np.abs(g - o)
        bad = err > rtol * a + 1e-30
        assert not bad.any(), f"row {r}: {bad.sum()} scores off, worst {err[bad].max()} vs A {a[bad][0]}"
        ratio = err / np.maximum(a, 1e-30)
        worst = max(worst, float(ratio.max()) if n else 0.0)
        big = np.abs(o) >= 1e-2 * a
        if big.any():
            rel = max(rel, float((err[big] / np.abs(o[big])).max()))
    return worst, rel


def recall(gpu_idx, want_idx):
    """Mean fraction of each row's wanted positions that the GPU selected."""
    fr = []
    for g, w in zip(gpu_idx, want_idx):
        ws = set(int(v) for v in w if v >= 0)
        if ws:
            fr.append(len(ws & set(int(v) for v in g if v >= 0)) / len(ws))
    return float(np.mean(fr)) if fr else 1.0


def check_mla(out_gpu, lse_gpu, out_ref, lse_ref, label=""):
    """The stated bars (max-abs 2e-2, mean-abs 5e-3) plus relative-RMS 1e-2 (whole) / 2e-2 (per row)
    and |dlse| <= 1e-3."""
    g = out_gpu.astype(np.float64)
    d = np.abs(g - out_ref)
    assert d.max() <= 2e-2, f"{label} max-abs {d.max()}"
    assert d.mean() <= 5e-3, f"{label} mean-abs {d.mean()}"
    ref_norm = np.linalg.norm(out_ref)
    if ref_norm > 0:
        rel = np.linalg.norm(g - out_ref) / ref_norm
        assert rel <= 1e-2, f"{label} relative RMS {rel}"
        rows_ref = np.linalg.norm(out_ref.reshape(out_ref.shape[0], -1), axis=1)
        rows_err = np.linalg.norm((g - out_ref).reshape(out_ref.shape[0], -1), axis=1)
        ok = rows_ref > 0
        if ok.any():
            assert (rows_err[ok] / rows_ref[ok]).max() <= 2e-2, f"{label} per-row relative RMS"
    else:
        rel = 0.0
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin), f"{label} lse finiteness"
        dl = np.abs(lse_gpu[fin].astype(np.float64) - lse_ref[fin])
        assert dl.size == 0 or dl.max() <= 1e-3, f"{label} lse {dl.max()}"
    return float(d.max()), float(d.mean()), float(rel)


def sets(idx):
    return [tuple(sorted(int(v) for v in row if v >= 0)) for row in idx]
