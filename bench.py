#!/usr/bin/env python3
"""DSA hot-path benchmark on one MI355X: tokens/s of dsa_forward (lightning indexer -> top-k ->
sparse MLA) on a seeded synthetic workload, with the roofline of the dominant stage and the CPU
oracle timed beside it.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one dsa_forward over the whole batch.  Inputs are resident in HBM before timing starts.
Each step is timed with HIP events on the stream the library launches on; the last-level cache
(256 MB MALL) and the L2s are flushed between steps (a 512 MiB read, outside the events), so that
gathered rows and cache pages come from HBM as they would in a model with many layers.  Rank 0 prints one JSON
line.  Only one GPU is supported: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}

WORKLOADS = {
    "tiny-prefill-L1024": lambda s: s.named_spec("tiny-prefill-L1024"),
    "decode-B64-ctx8192": lambda s: s.named_spec("decode-B64-ctx8192"),
    "prefill-L16384": lambda s: s.named_spec("prefill-L16384"),
    "mtp-decode-B32x2-ctx65536-paged": lambda s: s.named_spec("mtp-decode-B32x2-ctx65536-paged"),
    "ragged-decode-B16-paged": lambda s: s.named_spec("ragged-decode-B16-paged"),
    "decode-B64-ctx16384": lambda s: s.sweep_spec(16384),
    "decode-B64-ctx32768": lambda s: s.sweep_spec(32768),
    "decode-B64-ctx65536": lambda s: s.sweep_spec(65536),
    "decode-B64-ctx131072": lambda s: s.sweep_spec(131072),
}
DEFAULT_WORKLOAD = "decode-B64-ctx8192"
CPU_SAMPLE = {"tiny-prefill-L1024": 1024, "decode-B64-ctx8192": 64, "prefill-L16384": 48,
              "mtp-decode-B32x2-ctx65536-paged": 24, "ragged-decode-B16-paged": 16}

KERNEL_SOURCE = {"indexer": ("indexer.hip", "indexer_fp8.h"), "topk": ("topk.hip", "topk_core.h"),
                 "sparse_mla": ("sparse_mla.hip",), "write_path": ("cache_write.hip",),
                 "value_restore": ("value_restore.hip",),
                 "indexer_topk": ("indexer_topk.hip", "indexer_fp8.h", "topk_core.h", "topk.hip")}
VALUE_DH = 128   # value width per head used for the value-restore measurement

# Rotated spans used for the write-path measurement: the indexer key's first 64 of 128 dims, and
# the latent row's decoupled channel (the 64 dims after the 512 latent dims), adjacent pairs, base 1e4.
WRITE_K_ROPE = (0, 64, True, 10000.0)
WRITE_LAT_ROPE = (512, 64, True, 10000.0)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--no-flush", action="store_true", help="do not flush caches between steps")
    ap.add_argument("--prewarm-ms", type=float, default=50.0,
                    help="GPU work (cache-flush reads) run before the warm-up steps, so that the clocks have left "
                         "their idle state when timing starts (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle spot check before timing")
    ap.add_argument("--stage", default="all",
                    choices=["all", "forward", "indexer", "topk", "sparse_mla", "copy", "write_path",
                             "value_restore"],
                    help="profiling aid: run only this stage --steps times (no JSON line)")
    ap.add_argument("--window", type=int, default=0,
                    help="selection variant: add the last W positions of each query to its top-k (set union)")
    ap.add_argument("--dynamic-k", action="store_true",
                    help="selection variant: a per-query k, drawn uniformly from [k/2, k] (seed 7)")
    ap.add_argument("--value-restore", action="store_true",
                    help="measure the value up-projection after sparse MLA (d_h = 128) on the workload's query "
                         "tokens instead of the forward; prints its own JSON line")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the decode-B64-ctx131072 block that the default workload's line carries")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--long-context-only", action="store_true",
                    help="profiling aid: only the decode-B64-ctx131072 block (forward and stages, --steps each), "
                         "printed as its own JSON line")
    ap.add_argument("--write-path", action="store_true",
                    help="measure the cache write path (query rotation + key / latent append) of the workload's "
                         "query tokens instead of the forward; prints its own JSON line")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------------
# algorithmic work per launch


def algorithmic(p, stage, selected=None):
    """(bytes, flops) the method must move / compute for one launch of a stage.  selected: the number
    of selected positions of each query when a selection variant is used (else min(n, k))."""
    s = p.spec
    n = p.q_len.astype(np.int64)
    k = s.topk
    HI, H = s.idx_heads, s.mla_heads
    long_ = n > k
    if stage == "indexer":
        # the measured call, dsa_indexer_scores: every query scored over its n positions and every
        # entry of its row written (-inf over [n, ld)); the forward's own indexer pass skips rows
        # with n <= k (all their positions are selected) and the masked entries
        elt = {"f32": 4, "bf16": 2, "fp8": 1}[s.idx_dtype]
        kscale = 4 if s.idx_dtype == "fp8" else 0
        ld = (int(p.max_len) + 63) // 64 * 64
        # key cache read once per sequence (up to its longest query)
        nmax_seq = np.zeros(s.B, np.int64)
        np.maximum.at(nmax_seq, p.q_seq, n)
        kbytes = int(nmax_seq.sum()) * (128 * elt + kscale)
        qbytes = s.T * HI * (128 * elt + 4 + (4 if s.idx_dtype == "fp8" else 0))
        sbytes = s.T * ld * 4
        flops = int(n.sum()) * HI * 128 * 2
        return kbytes + qbytes + sbytes, flops
    if stage == "topk":
        if selected is not None:
            return int(n.sum()) * 4 + int(selected.sum()) * 4, 0
        return int(n[long_].sum()) * 4 + s.T * k * 4, 0
    if stage == "write_path":
        # every query token: its indexer key and latent row appended (sources bf16), its query
        # block rotated (indexer q bf16 -> the workload's indexer dtype; MLA q: the 64-dim span of
        # each head read and written in place); plus the seq / pos arrays
        elt = {"f32": 4, "bf16": 2, "fp8": 1}[s.idx_dtype]
        fp8s = 4 if s.idx_dtype == "fp8" else 0
        append = 128 * 2 + 576 * 2 + 8 + 128 * elt + fp8s + 576 * 2
        queries = 4 + HI * (128 * 2 + 128 * elt + fp8s) + H * 64 * 2 * 2
        return s.T * (append + queries), 0
    if stage == "sparse_mla":
        cnt = np.minimum(n, k) if selected is None else selected.astype(np.int64)
        gather = int(cnt.sum()) * (576 * 2 + 4)
        qo = s.T * H * (576 * 2 + 512 * 2 + 4)
        flops = int(cnt.sum()) * H * (576 + 512) * 2
        return gather + qo, flops
    raise ValueError(stage)


def bound_of(p, stage):
    if stage == "indexer" and p.spec.idx_dtype != "fp8" and p.spec.B == 1 and p.spec.T > 256:
        return "mfma", "bf16"
    if stage == "sparse_mla" and p.spec.B == 1 and p.spec.T > 256:
        return "mfma", "bf16"
    return "hbm", None


def source_hash(stage):
    """sha256/16 over the stage's kernel sources, then common.h."""
    csrc = os.path.join(ROOT, "sparse_attention_sum_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCE[stage] + ("common.h",):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(stage, workload):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(f"{stage}@{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(stage):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def achievable_peaks(dev, stream):
    """What this GPU delivers, measured with the probe kernels (probe/libpeaks.so): a streaming read
    of 4 GiB (GB/s) and a bf16 MFMA loop (TFLOP/s), best of 5 launches each, HIP events on `stream`."""
    import ctypes
    import torch
    from sparse_attention_sum_amd import build as libbuild
    L = ctypes.CDLL(libbuild.PROBE_LIB)
    L.peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.peak_read.restype = L.peak_mfma_bf16.restype = ctypes.c_int
    st = ctypes.c_void_p(stream.cuda_stream)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    read_blocks, mfma_blocks, iters = 256 * 16, 256 * 2, 20000
    sink = torch.empty(read_blocks * 256, dtype=torch.int32, device=dev)

    def best(fn):
        ts = []
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = fn()
            e1.record(stream)
            assert rc == 0, f"probe launch failed ({rc})"
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts[1:])

    t_read = best(lambda: L.peak_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                      read_blocks, st))
    t_mfma = best(lambda: L.peak_mfma_bf16(iters, ctypes.c_void_p(sink.data_ptr()), mfma_blocks, st))
    del buf
    flops = mfma_blocks * 4 * iters * 4 * 32768
    return {"hbm_read_GBs": round(nbytes / t_read / 1e9, 1), "bf16_mfma_TFLOPs": round(flops / t_mfma / 1e12, 1),
            "method": "streaming read of 4 GiB (16-byte loads, 8 in flight per thread) and a loop of "
                      "independent 32x32x16 bf16 MFMA chains at 2 waves per SIMD; best of 5"}


def long_context_block(dev, stream, flush, timed, steps=10, prewarm=None):
    """The batched-decode shape at 131072 positions (64 sequences, one query each), drawn on the
    device: forward and per-stage times, the sparse-MLA stage's HBM fraction, and a spot check of two
    queries against the oracle (indexer scores, the top-k set on the GPU's scores, sparse MLA on the
    GPU's indices)."""
    import torch
    import oracle
    from sparse_attention_sum_amd import dsa, synth

    ctx, T, H, k = 131072, 64, 128, 2048
    t0 = time.time()
    d = synth.build_decode_on_device(ctx, T, seed=1, device=dev)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    b = dsa.Batch(cu_q=d["cu_q"], q_seq=d["q_seq"], q_len=d["q_len"], max_len=ctx, max_q=1)
    kc = dsa.Cache(d["k_idx"], d["k_idx_scale"], seq_stride=ctx)
    lc = dsa.Cache(d["latent"], seq_stride=ctx)
    scale = 1.0 / 24.0
    ld = dsa.score_ld(b)
    scores = torch.empty((T, ld), dtype=torch.float32, device=dev)
    ind = torch.empty((T, k), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, dsa.dsa_workspace_size(dsa.DSA_OP_FORWARD, b, k, H)), dtype=torch.uint8, device=dev)
    tk_ws_n = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, b, k, H)
    tk_ws = torch.empty(max(1, tk_ws_n), dtype=torch.uint8, device=dev)
    mla_ws = torch.empty(max(1, dsa.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, b, k, H)), dtype=torch.uint8,
                         device=dev)
    fwd = lambda: dsa.dsa_forward(d["q_idx"], d["q_idx_scale"], d["w"], kc, k, d["q_mla"], lc, b, scale,
                                  indices_out=ind, out=out, lse=lse, workspace=ws, stream=stream)
    it_ws = torch.empty(max(1, dsa.dsa_workspace_size(dsa.DSA_OP_INDEXER_TOPK, b, k, H)), dtype=torch.uint8,
                        device=dev)
    stage = {
        "indexer_topk_fused": lambda: dsa.dsa_indexer_topk(d["q_idx"], d["q_idx_scale"], d["w"], kc, b, k,
                                                           indices=ind, workspace=it_ws, stream=stream),
        "indexer": lambda: dsa.dsa_indexer_scores(d["q_idx"], d["q_idx_scale"], d["w"], kc, b, 1.0, scores=scores,
                                                  ld=ld, stream=stream),
        "topk": lambda: dsa.dsa_topk(scores, ld, b, k, indices=ind, stream=stream, workspace=tk_ws),
        "sparse_mla": lambda: dsa.dsa_sparse_mla(d["q_mla"], lc, b, ind, scale, out=out, lse=lse, workspace=mla_ws,
                                                 stream=stream),
    }
    if prewarm is not None:
        prewarm(50.0)
    for _ in range(3):   # warm-up steps shaped like the timed ones (flush, then the forward)
        flush()
        fwd()
    torch.cuda.synchronize()
    ms, _ = timed(fwd, steps)
    res = {"workload": "decode-B64-ctx131072 (inputs drawn on the device)", "steps": steps,
           "ms_per_step": round(float(ms.mean()), 5), "median_ms": round(float(np.median(ms)), 5),
           "tokens_per_s": round(T / (float(ms.mean()) / 1e3), 1),
           "step_ms": [round(float(x), 4) for x in ms],
           "stages_us": {}, "setup_s": round(gen_s, 1)}
    for name in ("indexer_topk_fused", "indexer", "topk", "sparse_mla"):
        stage[name]()
        sms, _ = timed(stage[name], steps)
        res["stages_us"][name] = round(float(sms.mean() * 1e3), 3)
    mla_bytes = T * k * (576 * 2 + 4) + T * H * (576 * 2 + 512 * 2 + 4)
    idx_bytes = T * ctx * (128 + 4) + T * 64 * (128 + 8) + T * ctx * 4
    fused_bytes = T * ctx * (128 + 4) + T * 64 * (128 + 8) + T * k * 4
    res["sparse_mla_hbm_frac"] = round(mla_bytes / (res["stages_us"]["sparse_mla"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    res["indexer_hbm_frac"] = round(idx_bytes / (res["stages_us"]["indexer"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    res["indexer_topk_fused_hbm_frac"] = round(
        fused_bytes / (res["stages_us"]["indexer_topk_fused"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    res["indexer_topk_fused_alg_bytes"] = fused_bytes
    res["indexer_topk_fused_traffic"] = recorded_traffic("indexer_topk", "decode-B64-ctx131072")
    # spot check of queries 0 and 63 against the oracle (their sequences copied to the host)
    torch.cuda.synchronize()
    check = {}
    for t in (0, 63):
        kq = d["q_idx"][t:t + 1].view(torch.uint8).cpu().numpy()
        qs = d["q_idx_scale"][t:t + 1].cpu().numpy()
        wt = d["w"][t:t + 1].cpu().numpy()
        krows = d["k_idx"][t * ctx:(t + 1) * ctx].view(torch.uint8).cpu().numpy()
        ksc = d["k_idx_scale"][t * ctx:(t + 1) * ctx].cpu().numpy()
        one = dict(q_seq=np.zeros(1, np.int32), q_len=np.array([ctx], np.int32), seq_stride=ctx, nthreads=16)
        ref = oracle.indexer(kq, "fp8", qs, wt, krows, "fp8", ksc, **one)
        A = oracle.indexer(kq & np.uint8(0x7F), "fp8", qs, np.abs(wt), krows & np.uint8(0x7F), "fp8", ksc, **one)
        g = scores[t, :ctx].double().cpu().numpy()
        idx_err = float((np.abs(g - ref[0, :ctx]) / np.maximum(A[0, :ctx], 1e-30)).max())
        assert idx_err <= 2e-2, f"long-context spot check: indexer |err|/A {idx_err}"
        gi = ind[t].cpu().numpy()
        want = oracle.topk(g[None], np.array([ctx], np.int32), k)[0]
        assert sorted(gi[gi >= 0].tolist()) == sorted(want[want >= 0].tolist()), "long-context spot check: top-k"
        sel = torch.from_numpy(gi.astype(np.int64)).to(dev) + t * ctx
        lat = d["latent"][sel].view(torch.int16).cpu().numpy().view(np.uint16)
        qm = d["q_mla"][t:t + 1].view(torch.int16).cpu().numpy().view(np.uint16)
        o_ref, _ = oracle.sparse_mla(qm, lat, np.zeros(1, np.int32), np.array([k], np.int32),
                                     np.arange(k, dtype=np.int32)[None], seq_stride=k, softmax_scale=scale,
                                     nthreads=16)
        mla_err = float(np.abs(out[t].float().cpu().numpy() - o_ref[0]).max())
        assert mla_err <= 2e-2, f"long-context spot check: sparse MLA max-abs {mla_err}"
        check[f"query{t}"] = {"indexer_err_over_A": idx_err, "topk": "bit-exact", "mla_max_abs": mla_err}
    res["spot_check"] = check
    del d, ws, scores
    torch.cuda.empty_cache()
    return res


def long_context_only(args, dev):
    import torch
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty(1, dtype=torch.float32, device=dev)

    def flush():
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:   # torch creates an event's HIP event at its first record: not inside a step
            e0.record(stream)
            e1.record(stream)
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        for e0, e1 in ev:
            flush()
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        gc.enable()
        return np.array([e0.elapsed_time(e1) for e0, e1 in ev]), None

    def prewarm(ms):
        for _ in range(max(1, int(ms / 0.14))):
            torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)

    print(json.dumps(long_context_block(dev, stream, flush, timed, steps=args.steps,
                                        prewarm=prewarm if args.prewarm_ms > 0 else None)), flush=True)


# ---------------------------------------------------------------------------------------------


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the DSA path here is a single-GPU kernel library", file=sys.stderr)
        sys.exit(2)

    import torch
    import oracle
    from sparse_attention_sum_amd import dsa, synth
    from sparse_attention_sum_amd.device import to_device

    dsa.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.long_context_only:
        return long_context_only(args, dev)
    spec = WORKLOADS[args.workload](synth)
    t_gen = time.time()
    p = synth.build(spec)
    dp = to_device(p, dev)
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    T, H, k = spec.T, spec.mla_heads, spec.topk
    b = dp.batch
    ld = dsa.score_ld(b)
    stream = torch.cuda.current_stream()

    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    variant = args.window > 0 or args.dynamic_k
    width = k + args.window
    kq = None
    if args.dynamic_k:
        kq_np = np.random.default_rng(7).integers(k // 2, k + 1, T).astype(np.int32)
        kq = torch.from_numpy(kq_np).to(dev)
    ind = torch.empty((T, width), dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, dsa.dsa_workspace_size(dsa.DSA_OP_FORWARD, b, k, H)), dtype=torch.uint8, device=dev)
    scores = torch.empty((T, ld), dtype=torch.float32, device=dev)
    mla_ws_n = dsa.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, b, width, H)
    mla_ws = torch.empty(max(1, mla_ws_n), dtype=torch.uint8, device=dev)

    if args.write_path or args.stage == "write_path":
        return write_path_bench(args, spec, p, dp, dev, stream)
    if args.value_restore or args.stage == "value_restore":
        return value_restore_bench(args, spec, p, dev, stream)

    def forward():
        if variant:
            # selection variant: the three steps through their own entry points
            dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, spec.idx_scale, scores=scores,
                                   ld=ld, stream=stream)
            dsa.dsa_topk_select(scores, ld, b, k, kq, args.window, indices=ind, stream=stream)
            dsa.dsa_sparse_mla(dp.q_mla, dp.latent, b, ind, spec.softmax_scale, out=out, lse=lse,
                               workspace=mla_ws if mla_ws_n else None, stream=stream)
            return
        dsa.dsa_forward(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, k, dp.q_mla, dp.latent, b, spec.softmax_scale,
                        idx_scale=spec.idx_scale, indices_out=ind, out=out, lse=lse, workspace=ws, stream=stream)

    def stage_fn(stage):
        if stage == "indexer":
            return lambda: dsa.dsa_indexer_scores(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, b, spec.idx_scale,
                                                   scores=scores, ld=ld, stream=stream)
        if stage == "topk":
            if variant:
                return lambda: dsa.dsa_topk_select(scores, ld, b, k, kq, args.window, indices=ind, stream=stream)
            return lambda: dsa.dsa_topk(scores, ld, b, k, indices=ind, stream=stream)
        if stage == "sparse_mla":
            return lambda: dsa.dsa_sparse_mla(dp.q_mla, dp.latent, b, ind, spec.softmax_scale, out=out, lse=lse,
                                              workspace=mla_ws if mla_ws_n else None, stream=stream)
        return forward

    flush_buf = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty(1, dtype=torch.float32, device=dev)

    def flush():
        # Read 512 MiB (more than the 256 MB MALL plus the L2s) so the step starts with caches
        # holding only clean, unrelated lines.  A write-based flush would leave dirty lines whose
        # write-back then competes with the step's own reads.
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)

    def prewarm(ms):
        # the GPU sits idle while inputs are built and checked on the host; a few tens of ms of
        # streaming reads bring its clocks up before the warm-up steps (untimed, nothing is kept)
        if ms > 0:
            n = max(1, int(ms / 0.14))   # one flush read takes about 0.14 ms
            for _ in range(n):
                torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:   # torch creates an event's HIP event at its first record: not inside a step
            e0.record(stream)
            e1.record(stream)
        # no garbage-collection pass between a step's start event and its launches (a host stall
        # there would be timed as GPU time)
        gc.collect()
        gc.disable()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in ev:
            flush()
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gc.enable()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        return ms, wall

    # profiling aid: one stage only
    if args.stage != "all":
        if args.stage == "copy":
            src = torch.empty(2 ** 30 // 4, dtype=torch.float32, device=dev).fill_(1.0)
            dst = torch.empty_like(src)
            for _ in range(args.steps):
                dst.copy_(src)
            torch.cuda.synchronize()
            print(json.dumps({"stage": "copy", "bytes_read_per_launch": 2 ** 30, "bytes_written_per_launch": 2 ** 30}))
            return
        forward()
        if args.stage in ("topk", "sparse_mla"):
            stage_fn("indexer")()   # the score rows the top-k stage reads (the forward keeps its own)
            if args.stage == "sparse_mla":
                stage_fn("topk")()
        torch.cuda.synchronize()
        fn = stage_fn(args.stage)
        for _ in range(args.warmup):
            fn()
        ms, _ = timed(fn, args.steps)
        print(json.dumps({"stage": args.stage, "workload": args.workload, "mean_us": float(ms.mean() * 1e3)}))
        return

    # correctness gate: spot-check a few queries against the oracle before timing
    forward()
    torch.cuda.synchronize()
    check = None
    if not args.no_check:
        rows = np.unique(np.linspace(0, T - 1, num=min(T, 4)).astype(np.int32))
        gi = ind[torch.from_numpy(rows).long().to(dev)].cpu().numpy()
        o_ref, l_ref = oracle.sparse_mla(p.q_mla, p.latent, p.q_seq, p.q_len, gi, seq_stride=p.seq_stride,
                                         page_table=p.page_table, page_size=spec.page_size,
                                         softmax_scale=spec.softmax_scale, qsel=rows, nthreads=8)
        o_gpu = out[torch.from_numpy(rows).long().to(dev)].float().cpu().numpy()
        err = float(np.abs(o_gpu - o_ref).max())
        assert err <= 2e-2, f"oracle spot check failed: max-abs {err}"
        check = {"rows": int(len(rows)), "mla_max_abs_err": err}

    prewarm(args.prewarm_ms)
    for _ in range(args.warmup):
        forward()
    ms, wall = timed(forward, args.steps)
    ms_per_step = float(ms.mean())
    value = T / (ms_per_step / 1e3)

    # per-stage timing through the separate entry points (same kernels, same launch shapes)
    stages = {}
    selected = (ind >= 0).sum(dim=1).cpu().numpy() if variant else None
    for st in ("indexer", "topk", "sparse_mla"):
        if st != "sparse_mla" and p.max_len <= k and not variant:
            continue
        fn = stage_fn(st)
        fn()
        sms, _ = timed(fn, max(5, min(args.steps, 30)))
        nbytes, flops = algorithmic(p, st, selected)
        stages[st] = {"mean_us": round(float(sms.mean() * 1e3), 3), "alg_bytes": nbytes, "alg_flops": flops}
    forward()   # leave the outputs of a full forward in place
    dom = max(stages, key=lambda s_: stages[s_]["mean_us"])
    d = stages[dom]
    bound, prec = bound_of(p, dom)
    traffic = None if variant else recorded_traffic(dom, args.workload)
    if bound == "hbm":
        achieved = d["alg_bytes"] / (d["mean_us"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        achieved = d["alg_flops"] / (d["mean_us"] * 1e-6) / 1e12
        peak = MFMA_PEAK_TFLOPS[prec]
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic}
    roofline["kernel"] = dom
    peaks = None
    if not args.no_peaks:
        peaks = achievable_peaks(dev, stream)
        ach = peaks["hbm_read_GBs"] if bound == "hbm" else peaks["bf16_mfma_TFLOPs"]
        roofline["achievable_peak"] = ach
        roofline["frac_of_achievable"] = round(achieved / ach, 4)
    for st, v in stages.items():
        v["hbm_GBs"] = round(v["alg_bytes"] / (v["mean_us"] * 1e-6) / 1e9, 1)
        if v["alg_flops"]:
            v["TFLOPs"] = round(v["alg_flops"] / (v["mean_us"] * 1e-6) / 1e12, 1)

    # CPU baseline: the oracle, untuned, on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        nsample = min(T, CPU_SAMPLE.get(args.workload, 16))
        rows = np.unique(np.linspace(0, T - 1, num=nsample).astype(np.int32))
        threads = min(16, len(os.sched_getaffinity(0)))
        # repeat the sample until about 5 s of CPU work have been timed (a steadier figure when
        # one pass is short); every repetition is the same, full oracle forward
        reps, t0 = 0, time.perf_counter()
        while True:
            if variant:
                osc = oracle.indexer(p.q_idx, spec.idx_dtype, p.q_idx_scale, p.w, p.k_idx, spec.idx_dtype,
                                     p.k_idx_scale, p.q_seq, p.q_len, seq_stride=p.seq_stride,
                                     page_table=p.page_table, page_size=spec.page_size, scale=spec.idx_scale,
                                     qsel=rows, nthreads=threads)
                osel = oracle.topk_select(osc, p.q_len[rows], k, None if kq is None else kq_np[rows], args.window,
                                          nthreads=threads)
                oracle.sparse_mla(p.q_mla, p.latent, p.q_seq, p.q_len, osel, seq_stride=p.seq_stride,
                                  page_table=p.page_table, page_size=spec.page_size,
                                  softmax_scale=spec.softmax_scale, qsel=rows, nthreads=threads)
            else:
                oracle.forward(p.q_idx, spec.idx_dtype, p.q_idx_scale, p.w, p.k_idx, spec.idx_dtype, p.k_idx_scale,
                               p.q_mla, p.latent, p.q_seq, p.q_len, k, seq_stride=p.seq_stride,
                               page_table=p.page_table, page_size=spec.page_size, scale=spec.idx_scale,
                               softmax_scale=spec.softmax_scale, qsel=rows, nthreads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 5.0 or reps >= 50:
                break
        cpu = {"value": round(reps * len(rows) / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{len(rows)} of {T} query tokens of {args.workload} (evenly spaced), fp64 oracle forward, "
                         f"{reps} repetition(s) in {dt:.2f} s wall", "cpu_model": cpu_model()}

    long_ctx = None
    if args.workload == DEFAULT_WORKLOAD and not args.no_long_context and not variant:
        long_ctx = long_context_block(dev, stream, flush, timed, prewarm=prewarm if args.prewarm_ms > 0 else None)

    line = {
        "metric": "DSA tokens/s (indexer+top-k+sparse MLA)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload + (f"+window{args.window}" if args.window else "")
                               + ("+dynamic-k" if args.dynamic_k else ""), "query_tokens": T, "sequences": spec.B,
                   "max_context": int(p.max_len), "topk": k, "indexer_heads": spec.idx_heads,
                   "indexer_dtype": {"fp8": "fp8_e4m3", "bf16": "bf16", "f32": "f32"}[spec.idx_dtype],
                   "mla_heads": H, "latent": "bf16 576/512", "paged": spec.paged,
                   "cache_state": "hot" if args.no_flush else "flushed between steps"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages_us": stages,
        "achievable_peaks": peaks,
        "decode_ctx131072": long_ctx,
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "median_ms": round(float(np.median(ms)), 5),
        "p10_p90_ms": [round(float(np.percentile(ms, 10)), 5), round(float(np.percentile(ms, 90)), 5)],
        "step_ms": [round(float(x), 4) for x in ms],
        "spot_check": check,
        "setup_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def value_restore_bench(args, spec, p, dev, stream):
    """Each head's value up-projection of the latent attention output for the workload's query
    tokens (o [T, H, 512] -> out [T, H, 128], W [H, 128, 512], synthetic bf16)."""
    import torch
    import oracle
    from sparse_attention_sum_amd import dsa

    T, H, dh = spec.T, spec.mla_heads, VALUE_DH
    g = torch.Generator(device=dev).manual_seed(99)
    o = (torch.randn((T, H, 512), generator=g, device=dev) / 24).to(torch.bfloat16)
    w = (torch.randn((H, dh, 512), generator=g, device=dev) / 22.6).to(torch.bfloat16)
    out = torch.empty((T, H, dh), dtype=torch.bfloat16, device=dev)
    step = lambda: dsa.dsa_value_restore(o, w, out=out, stream=stream)
    flush_buf = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty(1, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:   # torch creates an event's HIP event at its first record: not inside a step
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    for e0, e1 in ev:
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    us = float(ms.mean() * 1e3)
    if args.stage == "value_restore":
        print(json.dumps({"stage": "value_restore", "workload": args.workload, "mean_us": us}))
        return
    nbytes = T * H * 512 * 2 + H * dh * 512 * 2 + T * H * dh * 2
    flops = 2 * T * H * 512 * dh
    # arithmetic intensity below the bf16 ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/B): HBM-bound
    if flops / nbytes < MFMA_PEAK_TFLOPS["bf16"] / HBM_PEAK_GBS * 1e3:
        achieved = nbytes / (us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = flops / (us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS["bf16"],
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS["bf16"], 4)}
    roofline["traffic"] = recorded_traffic("value_restore", args.workload)
    roofline["kernel"] = "value_restore"
    cpu = None
    if not args.no_cpu_baseline:
        rows = np.unique(np.linspace(0, T - 1, num=min(T, 8)).astype(np.int64))
        ob = o[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
        wb = w.view(torch.int16).cpu().numpy().view(np.uint16)
        threads = min(16, len(os.sched_getaffinity(0)))
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.value_restore(ob, wb, nthreads=threads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 5.0 or reps >= 100:
                break
        cpu = {"value": round(reps * len(rows) / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{len(rows)} of {T} tokens (evenly spaced), fp64 oracle, {reps} repetition(s) in {dt:.2f} s"}
    line = {
        "metric": "value restore tokens/s (per-head up-projection of the latent attention output)",
        "value": round(T / (us * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "heads": H, "latent": 512, "d_h": dh,
                   "cache_state": "hot" if args.no_flush else "flushed between steps"},
        "roofline": roofline, "cpu_baseline": cpu, "alg_bytes": nbytes, "alg_flops": flops,
        "median_ms": round(float(np.median(ms)), 5),
        "p10_p90_ms": [round(float(np.percentile(ms, 10)), 5), round(float(np.percentile(ms, 90)), 5)],
    }
    print(json.dumps(line), flush=True)


def write_path_bench(args, spec, p, dp, dev, stream):
    """The cache write path for the workload's query tokens: dsa_rope_queries (indexer q to the
    workload's indexer dtype, MLA q rotated in place) + dsa_cache_append (indexer key and latent row
    of each token, at its position)."""
    import torch
    import oracle
    from sparse_attention_sum_amd import dsa

    T, HI, H = spec.T, spec.idx_heads, spec.mla_heads
    g = torch.Generator(device=dev).manual_seed(1234)
    seq = torch.from_numpy(p.q_seq.astype(np.int32)).to(dev)
    pos = torch.from_numpy((p.q_len - 1).astype(np.int32)).to(dev)
    k_new = torch.randn((T, 128), generator=g, device=dev).to(torch.bfloat16)
    lat_new = (torch.randn((T, 576), generator=g, device=dev) / 24).to(torch.bfloat16)
    qi_in = torch.randn((T, HI, 128), generator=g, device=dev).to(torch.bfloat16)
    odt = {"fp8": torch.uint8, "bf16": torch.int16, "f32": torch.float32}[spec.idx_dtype]
    qi_out = torch.empty((T, HI, 128), dtype=odt, device=dev)
    qi_scale = torch.empty((T, HI), dtype=torch.float32, device=dev) if spec.idx_dtype == "fp8" else None
    qm = dp.q_mla.clone()
    # the caches of the workload (copies: the forward inputs stay as they are)
    kc = dsa.Cache(dp.k_cache.data.clone(), None if dp.k_cache.scale is None else dp.k_cache.scale.clone(),
                   seq_stride=dp.k_cache.seq_stride, page_table=dp.k_cache.page_table, page_size=dp.k_cache.page_size,
                   dtype=dp.k_cache.dtype)
    lc = dsa.Cache(dp.latent.data.clone(), None, seq_stride=dp.latent.seq_stride, page_table=dp.latent.page_table,
                   page_size=dp.latent.page_size, dtype=dp.latent.dtype)
    kr, lr = dsa.Rope(*WRITE_K_ROPE), dsa.Rope(*WRITE_LAT_ROPE)

    def step():
        dsa.dsa_rope_queries(qi_in, qi_out, qi_scale, qm, pos, kr, lr, stream=stream)
        dsa.dsa_cache_append(k_new, lat_new, seq, pos, spec.B, kc, lc, kr, lr, stream=stream)

    flush_buf = torch.ones(512 * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty(1, dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in ev:   # torch creates an event's HIP event at its first record: not inside a step
        e0.record(stream)
        e1.record(stream)
    torch.cuda.synchronize()
    for e0, e1 in ev:
        if not args.no_flush:
            torch.sum(flush_buf, dim=0, keepdim=True, out=flush_out)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
    if args.stage == "write_path":
        print(json.dumps({"stage": "write_path", "workload": args.workload, "mean_us": float(ms.mean() * 1e3)}))
        return
    us = float(ms.mean() * 1e3)
    nbytes, _ = algorithmic(p, "write_path")
    achieved = nbytes / (us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic("write_path", args.workload),
                "kernel": "write_path"}
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's write functions on a bounded sample of the same tokens
        rows = np.unique(np.linspace(0, T - 1, num=min(T, 16)).astype(np.int64))
        rsel = torch.from_numpy(rows).to(dev)
        kx = k_new[rsel].view(torch.int16).cpu().numpy().view(np.uint16)
        lx = lat_new[rsel].view(torch.int16).cpu().numpy().view(np.uint16)
        qx = qi_in[rsel].view(torch.int16).cpu().numpy().view(np.uint16)
        qmx = qm[rsel].view(torch.int16).cpu().numpy().view(np.uint16)
        psel = (p.q_len[rows] - 1).astype(np.int32)
        krt = (WRITE_K_ROPE[0], WRITE_K_ROPE[1], int(WRITE_K_ROPE[2]), WRITE_K_ROPE[3])
        lrt = (WRITE_LAT_ROPE[0], WRITE_LAT_ROPE[1], int(WRITE_LAT_ROPE[2]), WRITE_LAT_ROPE[3])
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.rope_store(qx, "bf16", psel, krt, spec.idx_dtype)
            oracle.rope_store(qmx, "bf16", psel, lrt, "bf16")
            oracle.rope_store(kx[:, None], "bf16", psel, krt, spec.idx_dtype)
            oracle.rope_store(lx[:, None], "bf16", psel, lrt, "bf16")
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 5.0 or reps >= 200:
                break
        cpu = {"value": round(reps * len(rows) / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{len(rows)} of {T} tokens of {args.workload} (evenly spaced): the oracle's rotation and "
                         f"storage of each token's queries and cache rows, {reps} repetition(s) in {dt:.2f} s"}
    line = {
        "metric": "cache write path tokens/s (query rotation + key / latent append)",
        "value": round(T / (us * 1e-6), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "indexer_heads": HI, "mla_heads": H,
                   "indexer_out": spec.idx_dtype, "k_rope": list(WRITE_K_ROPE), "latent_rope": list(WRITE_LAT_ROPE),
                   "paged": spec.paged, "cache_state": "hot" if args.no_flush else "flushed between steps"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "alg_bytes": nbytes,
        "median_ms": round(float(np.median(ms)), 5),
        "p10_p90_ms": [round(float(np.percentile(ms, 10)), 5), round(float(np.percentile(ms, 90)), 5)],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
