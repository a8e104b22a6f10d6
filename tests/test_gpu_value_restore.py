"""GPU parity of dsa_value_restore (each head's value up-projection of the latent attention output,
MQA form) against the oracle: |gpu - oracle| <= 2^-8 |oracle| + 1e-4 * A, A = sum_k |o| |w| (one
bf16 rounding of the output plus fp32 accumulation over 512 terms)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import log
from sparse_attention_sum_amd import dsa

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check(o, w, got, rows=None, label=""):
    ob, wb = bits(o), bits(w)
    if rows is not None:
        ob = ob[rows]
    ref = oracle.value_restore(ob, wb, nthreads=8)
    A = oracle.value_restore(ob & 0x7fff, wb & 0x7fff, nthreads=8)     # |o| . |w|
    g = got.float().cpu().numpy()
    if rows is not None:
        g = g[rows]
    err = np.abs(g - ref)
    tol = 2.0 ** -8 * np.abs(ref) + 1e-4 * A
    assert np.all(err <= tol), f"{label}: max err {err.max():.3g}, worst ratio {(err / tol).max():.3g}"
    log(f"{label}: max err {err.max():.3g}, worst err/tol {(err / tol).max():.3g}")


@pytest.mark.parametrize("T,H,dh", [(64, 128, 128), (300, 8, 256), (1, 1, 512), (129, 16, 384)])
def test_value_restore_matches_oracle(T, H, dh):
    g = torch.Generator(device="cuda").manual_seed(T * 1000 + H + dh)
    log(f"case: value_restore T={T} H={H} dh={dh}")
    o = (torch.randn((T, H, 512), generator=g, device="cuda") / 24).to(torch.bfloat16)
    w = (torch.randn((H, dh, 512), generator=g, device="cuda") / 22.6).to(torch.bfloat16)
    out = dsa.dsa_value_restore(o, w)
    torch.cuda.synchronize()
    check(o, w, out, label=f"T={T} H={H} dh={dh}")


def test_value_restore_prefill_size_sampled():
    T, H, dh = 16384, 128, 128
    g = torch.Generator(device="cuda").manual_seed(7)
    log("case: value_restore 16384 x 128 heads, sampled tokens")
    o = (torch.randn((T, H, 512), generator=g, device="cuda") / 24).to(torch.bfloat16)
    w = (torch.randn((H, dh, 512), generator=g, device="cuda") / 22.6).to(torch.bfloat16)
    out = dsa.dsa_value_restore(o, w)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(8).choice(T, 24, replace=False))
    rt = torch.from_numpy(rows).cuda()
    check(o[rt], w, out[rt], label="prefill sampled")


def test_value_restore_identity_weights_are_exact():
    T, H, dh = 70, 4, 128
    o = (torch.randn((T, H, 512), device="cuda") / 24).to(torch.bfloat16)
    w = torch.zeros((H, dh, 512), device="cuda")
    for h in range(H):
        w[h, torch.arange(dh), 128 * h + torch.arange(dh)] = 1.0
    out = dsa.dsa_value_restore(o, w.to(torch.bfloat16))
    torch.cuda.synchronize()
    for h in range(H):
        assert torch.equal(out[:, h], o[:, h, 128 * h:128 * h + dh])
