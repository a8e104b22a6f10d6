"""Pins of the oracle's value restore (page "DeepSeek-V3.2加速技术详解", 3.1 "MHA版MLA VS MQA版MLA":
each head's value is restored from the latent attention output afterwards):
    out[t, h, n] = sum_k o[t, h, k] * W[h, n, k].

Pins: numpy's einsum on the decoded values, an identity-like W that copies the first d_h latent
dims exactly, per-head independence (a transposed operand or a head mix-up fails), linearity.
"""
import numpy as np
import torch

import oracle


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_matches_einsum():
    rng = np.random.default_rng(51)
    o = _bf16(rng.normal(0, 1, (5, 3, 512)))
    w = _bf16(rng.normal(0, 0.05, (3, 64, 512)))
    got = oracle.value_restore(o, w)
    ref = np.einsum("thk,hnk->thn", oracle.decode(o, "bf16"), oracle.decode(w, "bf16"))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_identity_weights_copy_latent_dims():
    rng = np.random.default_rng(52)
    o = _bf16(rng.normal(0, 1, (4, 2, 512)))
    w = np.zeros((2, 128, 512), np.float32)
    w[0, np.arange(128), np.arange(128)] = 1.0          # head 0: the first 128 dims
    w[1, np.arange(128), 384 + np.arange(128)] = 2.0    # head 1: twice the last 128 dims
    got = oracle.value_restore(o, _bf16(w))
    dec = oracle.decode(o, "bf16")
    assert np.array_equal(got[:, 0], dec[:, 0, :128])
    assert np.array_equal(got[:, 1], 2.0 * dec[:, 1, 384:])


def test_heads_independent_and_linear():
    rng = np.random.default_rng(53)
    o = _bf16(rng.normal(0, 1, (3, 4, 512)))
    w = rng.normal(0, 0.05, (4, 32, 512)).astype(np.float32)
    base = oracle.value_restore(o, _bf16(w))
    w2 = w.copy(); w2[2] = 0.0
    got = oracle.value_restore(o, _bf16(w2))
    assert np.all(got[:, 2] == 0) and np.array_equal(got[:, [0, 1, 3]], base[:, [0, 1, 3]])
    w3 = _bf16(w); w3d = oracle.decode(w3, "bf16") * 2       # doubling a bf16 value is exact
    got3 = oracle.value_restore(o, _bf16(w3d))
    np.testing.assert_allclose(got3, 2 * base, rtol=1e-12, atol=0)
