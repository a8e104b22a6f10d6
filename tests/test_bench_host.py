"""Host-side checks of bench.py (no GPU): the one-GPU contract and the algorithmic work that the
roofline figures divide by, recomputed here in closed form from the workload's definition."""
import os
import subprocess
import sys
import types

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sparse_attention_sum_amd import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def _stand_in(spec):
    """q_len / q_seq of a workload without building its tensors (each query sees its whole context)."""
    q_len = np.concatenate([np.arange(c - q + 1, c + 1) for c, q in zip(spec.ctx, spec.nq)]).astype(np.int32)
    q_seq = np.concatenate([np.full(q, b) for b, q in enumerate(spec.nq)]).astype(np.int32)
    return types.SimpleNamespace(spec=spec, q_len=q_len, q_seq=q_seq, max_len=int(max(spec.ctx)))


def test_decode_algorithmic_work_in_closed_form():
    p = _stand_in(synth.named_spec("decode-B64-ctx8192"))                 # 64 sequences x 8192, one query each, fp8 indexer
    T, n, HI, H, k = 64, 8192, 64, 128, 2048
    idx_bytes, idx_flops = bench.algorithmic(p, "indexer")
    # keys (128 fp8 + 4-byte scale) once per sequence, q (fp8 + weight + q scale) per head, f32 scores
    assert idx_bytes == T * n * 132 + T * HI * (128 + 4 + 4) + T * n * 4
    assert idx_flops == T * n * HI * 128 * 2
    tk_bytes, _ = bench.algorithmic(p, "topk")
    assert tk_bytes == T * n * 4 + T * k * 4
    mla_bytes, mla_flops = bench.algorithmic(p, "sparse_mla")
    # k selected rows of 576 bf16 (+ 4-byte index), q (576 bf16) and out (512 bf16) + lse per head
    assert mla_bytes == T * k * (1152 + 4) + T * H * (1152 + 1024 + 4)
    assert mla_flops == T * k * H * (576 + 512) * 2
    assert bench.bound_of(p, "sparse_mla") == ("hbm", None)


def test_prefill_indexer_call_scores_every_row_and_writes_the_mask():
    """The indexer stage is timed through dsa_indexer_scores: every causal row is scored and every
    entry of [0, ld) written (-inf past n), so its bytes hold the whole 16384 x 16384 score matrix."""
    p = _stand_in(synth.named_spec("prefill-L16384"))                 # one sequence, 16384 causal queries, bf16 indexer
    n = np.arange(1, 16385, dtype=np.int64)
    idx_bytes, idx_flops = bench.algorithmic(p, "indexer")
    assert idx_flops == int(n.sum()) * 64 * 128 * 2
    assert idx_bytes == 16384 * 256 + 16384 * 64 * (256 + 4) + 16384 * 16384 * 4
    _, mla_flops = bench.algorithmic(p, "sparse_mla")
    assert mla_flops == int(np.minimum(n, 2048).sum()) * 128 * 1088 * 2
    assert bench.bound_of(p, "indexer") == ("mfma", "bf16")
