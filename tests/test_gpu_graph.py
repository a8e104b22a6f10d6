"""dsa_forward_noalloc captured into a HIP graph (through torch.cuda.graph) and replayed: every replay
equals the eager call bit for bit, also with other eager forwards (which reuse the same static
scratch with other data) between the replays."""
import pytest
import torch

from helpers import log
from sparse_attention_sum_amd import dsa, synth
from sparse_attention_sum_amd.device import to_device

pytestmark = pytest.mark.gpu


def _call(dp, out, lse, ind):
    s = dp.spec
    dsa.dsa_forward_noalloc(dp.q_idx, dp.q_idx_scale, dp.w, dp.k_cache, s.topk, dp.q_mla, dp.latent, dp.batch,
                            s.softmax_scale, out, idx_scale=s.idx_scale, indices_out=ind, lse=lse)


def _outputs(dp):
    T, H, k = dp.spec.T, dp.spec.mla_heads, dp.spec.topk
    return (torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda"),
            torch.empty((T, H), dtype=torch.float32, device="cuda"),
            torch.empty((T, k), dtype=torch.int32, device="cuda"))


def test_noalloc_forward_replays_from_a_graph():
    # ragged paged decode: a row past 32768 (two-pass top-k), a two-token sequence, split attention
    dp = to_device(synth.build(synth.Spec("graph-1", ctx=[9000, 3000, 40000], nq=[1, 2, 1],
                                          idx_dtype=synth.FP8, paged=True, seed=71)))
    other = to_device(synth.build(synth.Spec("graph-2", ctx=[5000, 2500], nq=[1, 1], idx_dtype=synth.FP8,
                                             seed=72)))
    ref = _outputs(dp)
    _call(dp, *ref)
    torch.cuda.synchronize()
    got = _outputs(dp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(dp, *got)                      # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _call(dp, *got)
    torch.cuda.synchronize()
    oth = _outputs(other)
    for r in range(3):
        for x in got:
            x.zero_()
        _call(other, *oth)                   # eager work on the same scratch between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got[2], ref[2]), f"replay {r}: indices differ"
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), f"replay {r}: output differs"
        assert torch.equal(got[1], ref[1]), f"replay {r}: lse differs"
    log("dsa_forward_noalloc: 3 graph replays equal the eager call bit for bit")
