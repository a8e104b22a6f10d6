"""dsa_forward_noalloc (the forward over libdsa's static scratch, for callers that cannot allocate)
against dsa_forward with a caller workspace: identical bits, on two calls in a row, the second with a
smaller batch (the scratch then still holds the first call's data), plus a rejection past its size."""
import numpy as np
import pytest
import torch

from helpers import log
from sparse_attention_sum_amd import dsa, synth
from sparse_attention_sum_amd.device import to_device

pytestmark = pytest.mark.gpu

SCRATCH = 96 << 20


def _both(spec):
    p = synth.build(spec)
    dp = to_device(p)
    b, s = dp.batch, dp.spec
    T, H = s.T, s.mla_heads
    need = dsa.dsa_workspace_size(dsa.DSA_OP_FORWARD, b, s.topk, H)
    assert 0 < need <= SCRATCH
    res = []
    for fn in ("forward", "noalloc"):
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
        ind = torch.empty((T, s.topk), dtype=torch.int32, device="cuda")
        if fn == "forward":
            dsa.dsa_forward(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, s.topk, dp.q_mla, dp.latent, b,
                            s.softmax_scale, idx_scale=s.idx_scale, indices_out=ind, out=out, lse=lse)
        else:
            dsa.dsa_forward_noalloc(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, s.topk, dp.q_mla, dp.latent, b,
                                    s.softmax_scale, out, idx_scale=s.idx_scale, indices_out=ind, lse=lse)
        torch.cuda.synchronize()
        res.append((out, lse, ind))
    (o1, l1, i1), (o2, l2, i2) = res
    assert torch.equal(i1, i2), f"{spec.name}: indices differ"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{spec.name}: output differs"
    assert torch.equal(l1, l2), f"{spec.name}: lse differs"
    log(f"{spec.name}: noalloc == forward bit for bit (workspace {need / 2**20:.1f} MiB)")
    return need


def test_noalloc_forward_equals_forward_twice_then_smaller():
    # 1: ragged paged decode with rows past 32768 (two-pass top-k) and 16 splits in the attention
    big = synth.Spec("noalloc-1", ctx=[40000, 9000, 1500, 70000], nq=[1, 2, 1, 1], idx_dtype=synth.FP8,
                     paged=True, seed=61)
    # 2: a smaller contiguous batch that only partly overwrites what the first call left
    small = synth.Spec("noalloc-2", ctx=[3000, 2100], nq=[1, 1], idx_dtype=synth.FP8, seed=62)
    n1 = _both(big)
    n2 = _both(small)
    assert n2 < n1


def test_noalloc_rejects_a_batch_past_the_scratch():
    spec = synth.Spec("noalloc-big", ctx=[70000] * 8, nq=[40] * 8, idx_dtype=synth.FP8, seed=63)
    T, H = spec.T, spec.mla_heads
    p = synth.Problem(spec=spec, q_seq=np.repeat(np.arange(8, dtype=np.int32), 40),
                      q_len=np.full(T, 70000, np.int32), cu_q=np.arange(0, T + 1, 40, dtype=np.int32),
                      max_len=70000, max_q=40, q_idx=np.zeros((T, 64, 128), np.uint8),
                      q_idx_scale=np.ones((T, 64), np.float32), w=np.ones((T, 64), np.float32),
                      k_idx=np.zeros((8 * 70000, 128), np.uint8), k_idx_scale=np.ones(8 * 70000, np.float32),
                      q_mla=np.zeros((T, H, 576), np.uint16), latent=np.zeros((8 * 70000, 576), np.uint16),
                      seq_stride=70000, page_table=None)
    dp = to_device(p)
    assert dsa.dsa_workspace_size(dsa.DSA_OP_FORWARD, dp.batch, spec.topk, H) > SCRATCH
    out = torch.full((T, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_forward_noalloc(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, spec.topk, dp.q_mla, dp.latent,
                                dp.batch, spec.softmax_scale, out)
    assert e.value.status == dsa.DSA_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)          # nothing was launched
